"""C ABI: the library loads, exports every declared symbol, and validates arguments.

These run on the CPU: every call here fails validation (or is an empty problem),
and the library returns before it touches the HIP runtime, so no GPU is needed.
Fake device pointers are plain aligned integers that are never dereferenced.
"""
import os
import re
import subprocess

import pytest

import causal_attention_flash_amd as caf
from causal_attention_flash_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP, ALIAS, SCRATCH = range(9)
BF16, F32, F16 = bd.ATTN_BF16, bd.ATTN_F32, bd.ATTN_F16

# distinct, 16-byte aligned, far apart fake device addresses
P = [0x10_0000_0000 * (i + 1) for i in range(12)]


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = {}
    for m in re.finditer(r"^(?:const\s+)?[\w\s\*]+?\b(attn_\w+)\s*\(([^;]*?)\)\s*;", text, flags=re.M | re.S):
        name, args = m.group(1), m.group(2).strip()
        decls[name] = 0 if args in ("", "void") else args.count(",") + 1
    return decls


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.fail(f"{bd.LIB_PATH} not built: run `python -m causal_attention_flash_amd.build`")
    return bd.load_library()


def test_header_declares_the_boundary():
    decls = _declared_functions()
    assert set(decls) == {"attn_fwd", "attn_bwd_workspace_bytes", "attn_bwd", "attn_bwd_preprocess",
                          "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dq_delta", "attn_status_string",
                          "attn_fwd_gqa", "attn_bwd_gqa", "attn_bwd_gqa_workspace_bytes",
                          "attn_decode", "attn_decode_workspace_bytes", "attn_fwd_fp8qk",
                          "attn_bwd_atomic", "attn_bwd_atomic_workspace_bytes", "attn_clock_sample",
                          "attn_bwd_noalloc"}
    for name, nargs in decls.items():
        assert len(bd.SIGNATURES[name][1]) == nargs, name


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bd.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code in range(9):
        s = bd.status_string(code)
        assert isinstance(s, str) and s
    assert bd.status_string(99) == "unknown attn_status"
    assert bd.status_string(OK) == "ok"


def fwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=3, S=100, D=64, scale=0.125, causal=1, dtype=BF16)
    a.update(kw)
    return bd.c_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"], a["D"], a["scale"],
                         a["causal"], a["dtype"], 0)


def bwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8], ws=P[9],
             ws_bytes=2 * 3 * 100 * 4, B=2, H=3, S=100, D=64, scale=0.125, causal=1, dtype=BF16)
    a.update(kw)
    return bd.c_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"],
                         a["ws_bytes"], a["B"], a["H"], a["S"], a["D"], a["scale"], a["causal"], a["dtype"], 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL),
    (dict(S=-1), SHAPE), (dict(B=-2), SHAPE), (dict(H=-1), SHAPE),
    (dict(B=1 << 20, H=1 << 11, S=1), SHAPE),          # B*H*S = 2^31
    (dict(B=1, H=1, S=1 << 25, D=64), SHAPE),           # S*D = 2^31
    (dict(D=112), UNSUP), (dict(D=48), UNSUP), (dict(D=32), UNSUP), (dict(D=256), UNSUP),
    (dict(dtype=3), UNSUP), (dict(dtype=-1), UNSUP),
    (dict(causal=2), UNSUP), (dict(causal=-1), UNSUP),
    (dict(scale=0.0), UNSUP), (dict(scale=-0.5), UNSUP), (dict(scale=float("nan")), UNSUP),
    (dict(scale=float("inf")), UNSUP),
    (dict(q=P[0] + 8), ALIGN), (dict(lse=P[4] + 4), ALIGN), (dict(o=P[3] + 2), ALIGN),
    (dict(o=P[0]), ALIAS), (dict(lse=P[1] + 64), ALIAS), (dict(lse=P[3] + 16), ALIAS),
])
def test_fwd_validation(lib, kw, expect):
    assert fwd(**kw) == expect


# Each documented limit at its edge.  The size and scale checks run before the
# pointer checks, so with q = NULL a value the contract accepts returns
# ATTN_ERR_NULL (it passed) and one it rejects returns its own status; nothing
# is launched either way.
@pytest.mark.parametrize("kw,expect", [
    (dict(B=(1 << 31) - 1, H=1, S=1), NULL),             # B*H*S = 2^31 - 1: accepted
    (dict(B=1 << 31, H=1, S=1), SHAPE),                  # B*H*S = 2^31
    (dict(B=1, H=(1 << 31) - 1, S=1), NULL),
    (dict(B=1 << 16, H=1 << 15, S=1), SHAPE),            # 2^31 through the product B*H
    (dict(B=1, H=1, S=(1 << 25) - 1, D=64), NULL),       # S*D = 2^31 - 64: accepted
    (dict(B=1, H=1, S=1 << 25, D=64), SHAPE),            # S*D = 2^31
    (dict(B=1, H=1, S=(1 << 24) - 1, D=128), NULL),
    (dict(B=1, H=1, S=1 << 24, D=128), SHAPE),
    (dict(B=1, H=1, S=(1 << 31) // 80, D=80), NULL),     # largest S with S*80 < 2^31
    (dict(B=1, H=1, S=(1 << 31) // 80 + 1, D=80), SHAPE),
    (dict(scale=1.4e-45), NULL),                         # smallest positive float: accepted
    (dict(scale=3.4028234663852886e38), NULL),           # largest finite float
    (dict(scale=0.0), UNSUP), (dict(scale=-0.0), UNSUP), (dict(scale=-1.4e-45), UNSUP),
    (dict(scale=float("inf")), UNSUP), (dict(scale=float("nan")), UNSUP),
])
def test_documented_limits_at_their_edges(lib, kw, expect):
    assert fwd(q=0, **kw) == expect
    # the backward and the decode call apply the same limits (decode: L for S)
    assert bwd(q=0, ws_bytes=1 << 62, **kw) == expect
    dkw = {("L" if key == "S" else key): val for key, val in kw.items()}
    assert dec(q=0, Hkv=1, **dkw) == expect


def bwd_noalloc(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8],
             B=2, H=3, S=100, D=64, scale=0.125, causal=1, dtype=BF16)
    a.update(kw)
    return bd.c_attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                 a["B"], a["H"], a["S"], a["D"], a["scale"], a["causal"], a["dtype"], 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), NULL), (dict(dv=0), NULL), (dict(lse=0), NULL),
    (dict(D=72), UNSUP), (dict(scale=0.0), UNSUP), (dict(causal=3), UNSUP), (dict(S=-1), SHAPE),
    (dict(dq=P[0] + 8), ALIGN), (dict(dq=P[1]), ALIAS), (dict(dk=P[6]), ALIAS),
    # the scratch holds 2^21 query rows: at the limit the next check (NULL) is what fails
    (dict(B=1, H=1, S=1 << 21, q=0), NULL), (dict(B=4, H=1 << 9, S=1 << 10, q=0), NULL),
    (dict(B=1, H=1, S=(1 << 21) + 1), SCRATCH), (dict(B=3, H=1 << 10, S=1 << 10), SCRATCH),
    (dict(B=0, q=0, dq=0), OK),
])
def test_bwd_noalloc_validation(lib, kw, expect):
    assert bwd_noalloc(**kw) == expect
    assert f"#define ATTN_NOALLOC_MAX_ROWS (1 << 21)" in open(HEADER).read()


def test_clock_sample_validation(lib):
    limit = 4096  # ATTN_CLOCK_SAMPLE_MAX
    assert f"#define ATTN_CLOCK_SAMPLE_MAX {limit}" in open(HEADER).read()
    assert bd.c_attn_clock_sample(P[0], 0) == SHAPE
    assert bd.c_attn_clock_sample(P[0], -1) == SHAPE
    assert bd.c_attn_clock_sample(P[0], limit + 1) == SHAPE
    assert bd.c_attn_clock_sample(0, 8) == NULL
    assert bd.c_attn_clock_sample(0, limit) == NULL
    assert bd.c_attn_clock_sample(P[0] + 8, 8) == ALIGN


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(S=0), dict(B=0, q=0, k=0, v=0, o=0, lse=0)])
def test_fwd_empty_problem_is_ok_without_pointers(lib, kw):
    assert fwd(**kw) == OK


def test_fwd_empty_still_checks_the_supported_set(lib):
    assert fwd(B=0, D=112) == UNSUP
    assert fwd(B=0, dtype=7) == UNSUP
    assert fwd(B=0, S=-1) == SHAPE


def test_fwd_adjacent_buffers_do_not_alias(lib):
    # o placed exactly after q (B*H*S*D*2 bytes): touching, not overlapping.  Then the
    # call passes validation and would launch, so instead shrink lse onto q's tail.
    n = 2 * 3 * 100 * 64 * 2
    assert fwd(lse=P[0] + n - 16) == ALIAS


@pytest.mark.parametrize("kw,expect", [
    (dict(ws=0), WS), (dict(ws_bytes=2 * 3 * 100 * 4 - 1), WS), (dict(ws_bytes=0), WS),
    (dict(ws=P[9] + 4), ALIGN),
    (dict(ws=P[0]), ALIAS), (dict(dq=P[1]), ALIAS), (dict(dk=P[6]), ALIAS), (dict(dv=P[5]), ALIAS),
    (dict(o=0), NULL), (dict(do=0), NULL), (dict(dq=0), NULL),
    (dict(D=72), UNSUP), (dict(S=-3), SHAPE), (dict(scale=-1.0), UNSUP),
])
def test_bwd_validation(lib, kw, expect):
    assert bwd(**kw) == expect


def test_bwd_empty_is_ok(lib):
    assert bwd(S=0, ws=0, ws_bytes=0, q=0) == OK


def test_workspace_bytes(lib):
    assert bd.c_attn_bwd_workspace_bytes(2, 3, 100, 64, BF16) == 2 * 3 * 100 * 4
    assert bd.c_attn_bwd_workspace_bytes(1, 16, 8191, 128, BF16) == 16 * 8191 * 4
    assert bd.c_attn_bwd_workspace_bytes(1, 4, 128, 64, F32) == 4 * 128 * 4
    assert bd.c_attn_bwd_workspace_bytes(0, 3, 100, 64, BF16) == 0
    assert bd.c_attn_bwd_workspace_bytes(2, 3, 100, 80, BF16) == 2 * 3 * 100 * 4
    assert bd.c_attn_bwd_workspace_bytes(2, 3, 100, 64, F16) == 2 * 3 * 100 * 4
    assert bd.c_attn_bwd_workspace_bytes(2, 3, 100, 64, 3) == 0
    assert bd.c_attn_bwd_workspace_bytes(2, 3, 100, 112, BF16) == 0
    assert bd.c_attn_bwd_workspace_bytes(2, 3, -1, 64, BF16) == 0


def test_stage_entry_points_validate(lib):
    assert bd.c_attn_bwd_preprocess(P[0], P[1], 0, 2, 3, 100, 64, BF16) == NULL
    assert bd.c_attn_bwd_preprocess(P[0], P[1], P[0], 2, 3, 100, 64, BF16) == ALIAS
    assert bd.c_attn_bwd_preprocess(P[0], P[1], P[2], 2, 3, 100, 48, BF16) == UNSUP
    assert bd.c_attn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[6], 2, 3, 100, 64, 0.1, 1, BF16) == ALIAS
    assert bd.c_attn_bwd_dkdv(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], 2, 3, 100, 64, 0.1, 3, BF16) == UNSUP
    assert bd.c_attn_bwd_dq(P[0], P[1], P[2], P[3], P[4], 0, P[6], 2, 3, 100, 64, 0.1, 1, BF16) == NULL
    assert bd.c_attn_bwd_dq(P[0], P[1], P[2], P[3], P[4], P[5], P[4] + 32, 2, 3, 100, 64, 0.1, 1, BF16) == ALIAS
    # attn_bwd_dq_delta(q, k, v, o, dout, lse, delta, dq, ...): delta and dq are outputs
    assert bd.c_attn_bwd_dq_delta(P[0], P[1], P[2], P[3], P[4], P[5], 0, P[7], 2, 3, 100, 64, 0.1, 1, BF16) == NULL
    assert bd.c_attn_bwd_dq_delta(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[3], 2, 3, 100, 64, 0.1, 1, BF16) == ALIAS
    assert bd.c_attn_bwd_dq_delta(P[0], P[1], P[2], P[3], P[4], P[5], P[5] + 64, P[7], 2, 3, 100, 64, 0.1, 1,
                                  BF16) == ALIAS
    assert bd.c_attn_bwd_dq_delta(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], 2, 3, 100, 64, 0.0, 1, BF16) == UNSUP
    assert bd.c_attn_bwd_dq_delta(P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], 0, 3, 100, 64, 0.1, 1, BF16) == OK


def test_torch_wrapper_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        caf.attn_fwd(q, q, q)


def test_missing_library_fails_loudly(tmp_path):
    saved = bd._lib
    bd._lib = None
    try:
        with pytest.raises(ImportError, match="no fallback"):
            bd.load_library(str(tmp_path / "nope.so"))
    finally:
        bd._lib = saved


# ------------------------------------------------------ grouped key/value heads


def fwd_gqa(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=8, Hkv=2, S=100, D=64, scale=0.125, causal=1,
             dtype=BF16)
    a.update(kw)
    return bd.c_attn_fwd_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["S"], a["D"],
                             a["scale"], a["causal"], a["dtype"], 0)


GQA_WS = 6400 + 2 * 409600  # delta 2*8*100*4 bytes, then fp32 dK and dV partials 2*8*100*64*4 bytes each


def bwd_gqa(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8], ws=P[9],
             ws_bytes=GQA_WS, B=2, H=8, Hkv=2, S=100, D=64, scale=0.125, causal=1, dtype=BF16)
    a.update(kw)
    return bd.c_attn_bwd_gqa(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"],
                             a["ws_bytes"], a["B"], a["H"], a["Hkv"], a["S"], a["D"], a["scale"], a["causal"],
                             a["dtype"], 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(Hkv=0), SHAPE), (dict(Hkv=3), SHAPE), (dict(Hkv=16), SHAPE), (dict(Hkv=-1), SHAPE),
    (dict(k=0), NULL), (dict(D=112), UNSUP), (dict(scale=0.0), UNSUP),
    # o overlapping the tail of k: K spans B*Hkv*S*D*2 = 51200 bytes (a call that
    # passes validation would launch, so only overlaps are checked here)
    (dict(o=P[1] + 51200 - 16), ALIAS), (dict(lse=P[2] + 51200 - 16), ALIAS),
])
def test_fwd_gqa_validation(lib, kw, expect):
    assert fwd_gqa(**kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(Hkv=0), SHAPE), (dict(Hkv=5), SHAPE), (dict(dk=0), NULL),
    (dict(ws_bytes=GQA_WS - 1), WS), (dict(ws=0), WS), (dict(ws=P[4] + 16), ALIAS),
    # dk overlapping dv: each spans B*Hkv*S*D*2 = 51200 bytes
    (dict(dv=P[7] + 51200 - 16), ALIAS), (dict(dk=P[5]), ALIAS),
])
def test_bwd_gqa_validation(lib, kw, expect):
    assert bwd_gqa(**kw) == expect


def test_gqa_workspace_bytes(lib):
    assert bd.c_attn_bwd_gqa_workspace_bytes(2, 8, 2, 100, 64, BF16) == GQA_WS
    assert bd.c_attn_bwd_gqa_workspace_bytes(2, 8, 8, 100, 64, BF16) == 2 * 8 * 100 * 4  # one per query head
    assert bd.c_attn_bwd_gqa_workspace_bytes(2, 8, 2, 100, 64, F32) == 2 * 8 * 100 * 4   # fp32 sums in-kernel
    assert bd.c_attn_bwd_gqa_workspace_bytes(2, 8, 3, 100, 64, BF16) == 0                # 3 does not divide 8
    assert bd.c_attn_bwd_gqa_workspace_bytes(0, 8, 2, 100, 64, BF16) == 0


def test_gqa_empty_problems_are_ok(lib):
    assert fwd_gqa(B=0, Hkv=0) == OK
    assert bwd_gqa(S=0) == OK
    assert fwd_gqa(B=0, Hkv=-1) == SHAPE


# ------------------------------------------------------------------- decode


def dec(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], lens=P[3], o=P[4], lse=P[5], ws=P[6], ws_bytes=1 << 30,
             B=8, H=16, Hkv=4, L=4096, D=64, scale=0.125, dtype=BF16)
    a.update(kw)
    return bd.c_attn_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["ws"], a["ws_bytes"], a["B"],
                            a["H"], a["Hkv"], a["L"], a["D"], a["scale"], a["dtype"], 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL),
    (dict(Hkv=3), SHAPE), (dict(Hkv=0), SHAPE), (dict(Hkv=-1), SHAPE), (dict(L=0), SHAPE), (dict(L=-1), SHAPE),
    (dict(B=-1), SHAPE), (dict(D=72), UNSUP), (dict(dtype=3), UNSUP), (dict(scale=0.0), UNSUP),
    (dict(q=P[0] + 8), ALIGN), (dict(lens=P[3] + 2), ALIGN), (dict(ws=P[6] + 8), ALIGN),
    (dict(ws=0), WS), (dict(ws_bytes=16), WS),
    (dict(o=P[1]), ALIAS), (dict(lse=P[0] + 64), ALIAS), (dict(ws=P[2] + 4096), ALIAS), (dict(o=P[3]), ALIAS),
])
def test_decode_validation(lib, kw, expect):
    assert dec(**kw) == expect


def test_decode_empty_and_workspace(lib):
    assert dec(B=0, q=0, k=0, v=0, o=0, lse=0, ws=0, ws_bytes=0) == OK
    assert dec(H=0, Hkv=0, ws=0, ws_bytes=0) == OK
    assert dec(B=0, L=0) == SHAPE
    # the workspace holds (D + 2) fp32 per query head and chunk; one chunk needs none
    nws = bd.c_attn_decode_workspace_bytes(8, 16, 4, 4096, 64, BF16)
    assert nws > 0 and nws % (8 * 16 * (64 + 2) * 4) == 0
    assert bd.c_attn_decode_workspace_bytes(8, 16, 4, 200, 64, BF16) == 0
    assert bd.c_attn_decode_workspace_bytes(8, 16, 3, 4096, 64, BF16) == 0
    assert bd.c_attn_decode_workspace_bytes(8, 16, 4, 4096, 72, BF16) == 0
    # with no workspace needed, a NULL workspace is accepted (the call then fails only
    # at launch, which the fake pointers would make unsafe: stop at validation)
    assert dec(L=200, ws=0, ws_bytes=0, q=P[0] + 8) == ALIGN


# --------------------------------------------------------- fp8 Q and K forward


def fwd8(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=8, Hkv=2, S=100, D=64, scale=0.125, qd=0.01,
             kd=0.02, causal=1, dtype=BF16)
    a.update(kw)
    return bd.c_attn_fwd_fp8qk(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["S"], a["D"],
                               a["scale"], a["qd"], a["kd"], a["causal"], a["dtype"], 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL),
    (dict(D=80), UNSUP), (dict(D=96), UNSUP), (dict(D=112), UNSUP), (dict(dtype=F32), UNSUP), (dict(dtype=3), UNSUP),
    (dict(scale=0.0), UNSUP), (dict(qd=0.0), UNSUP), (dict(kd=-1.0), UNSUP), (dict(qd=float("inf")), UNSUP),
    (dict(kd=float("nan")), UNSUP), (dict(qd=1e30, kd=1e30), UNSUP), (dict(causal=2), UNSUP),
    (dict(Hkv=3), SHAPE), (dict(Hkv=0), SHAPE), (dict(B=-1), SHAPE),
    (dict(q=P[0] + 8), ALIGN), (dict(k=P[1] + 4), ALIGN), (dict(lse=P[4] + 4), ALIGN),
    # K holds B*Hkv*S*D = 25600 bytes (one per code), V 51200 (bf16), O 102400
    (dict(o=P[1] + 25600 - 16), ALIAS), (dict(lse=P[2] + 51200 - 16), ALIAS), (dict(o=P[0] + 51200 - 16), ALIAS),
    (dict(lse=P[3] + 102400 - 16), ALIAS),
])
def test_fwd_fp8qk_validation(lib, kw, expect):
    assert fwd8(**kw) == expect


def test_fwd_fp8qk_empty_is_ok(lib):
    assert fwd8(B=0, q=0, k=0, v=0, o=0, lse=0) == OK
    assert fwd8(S=0) == OK
    assert fwd8(B=0, D=80) == UNSUP  # the supported set is checked even with nothing to do


# ------------------------------------------------------------- atomic-dQ backward


def bwda(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8], ws=P[9],
             ws_bytes=1 << 30, B=2, H=4, S=100, D=64, scale=0.125, causal=1, dtype=BF16)
    a.update(kw)
    return bd.c_attn_bwd_atomic(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["ws"],
                                a["ws_bytes"], a["B"], a["H"], a["S"], a["D"], a["scale"], a["causal"], a["dtype"], 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), NULL), (dict(dq=0), NULL), (dict(lse=0), NULL),
    (dict(D=128), UNSUP), (dict(D=80), UNSUP), (dict(dtype=F32), UNSUP), (dict(scale=-1.0), UNSUP),
    (dict(causal=5), UNSUP), (dict(B=-1), SHAPE),
    (dict(ws=0), WS), (dict(ws_bytes=16), WS), (dict(ws=P[9] + 8), ALIGN), (dict(dk=P[7] + 4), ALIGN),
    # dq overlapping q (each [B,H,S,D] bf16 = 51200 bytes), the workspace overlapping lse
    (dict(dq=P[0] + 51200 - 16), ALIAS), (dict(ws=P[5]), ALIAS), (dict(dv=P[6]), ALIAS),
])
def test_bwd_atomic_validation(lib, kw, expect):
    assert bwda(**kw) == expect


def test_bwd_atomic_workspace_and_empty(lib):
    # delta 2*4*100*4 = 3200 bytes rounded to 3328, then the fp32 dQ sums 2*4*100*64*4 bytes
    assert bd.c_attn_bwd_atomic_workspace_bytes(2, 4, 100, 64, BF16) == 3328 + 204800
    assert bd.c_attn_bwd_atomic_workspace_bytes(2, 4, 100, 128, BF16) == 0
    assert bd.c_attn_bwd_atomic_workspace_bytes(2, 4, 100, 64, F32) == 0
    assert bwda(B=0, q=0, ws=0, ws_bytes=0) == OK
    assert bwda(S=0, D=128) == UNSUP
