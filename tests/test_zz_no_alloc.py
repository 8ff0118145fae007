"""attn_bwd_noalloc through the C ABI (its delta lives in the library's static
scratch array): two calls in a row, the second on a smaller problem, each against
attn_bwd on the same inputs.  The same kernels run in the same order, so the
outputs must be bitwise equal (a stricter bar than the oracle tolerance)."""
import numpy as np
import pytest

import seeded_inputs as si
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    return gu.require_gpu()


def run_pair(w, device, seed):
    import causal_attention_flash_amd as caf
    from causal_attention_flash_amd import _binding as bd
    torch = gu.torch_mod()
    x = si.make_inputs(w, seed=seed)
    q, k, v, do = (gu.to_device(x, n, w.dtype, device) for n in ("q", "k", "v", "do"))
    o, lse = caf.attn_fwd(q, k, v, scale=w.scale, causal=w.causal)
    dt = {"bf16": bd.ATTN_BF16, "f16": bd.ATTN_F16, "f32": bd.ATTN_F32}[w.dtype]
    stream = torch.cuda.current_stream(device).cuda_stream
    B, H, S, D = q.shape
    ref = [torch.empty_like(q) for _ in range(3)]
    nws = bd.c_attn_bwd_workspace_bytes(B, H, S, D, dt)
    ws = torch.empty(nws, dtype=torch.uint8, device=device)
    st = bd.c_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                       *(t.data_ptr() for t in ref), ws.data_ptr(), nws, B, H, S, D, w.scale, int(w.causal), dt,
                       stream)
    assert st == 0, bd.status_string(st)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    st = bd.c_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), *(t.data_ptr() for t in got), B, H, S, D, w.scale, int(w.causal), dt,
                               stream)
    assert st == 0, bd.status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype != torch.float32 else b.view(torch.int32)), name
    return [gu.to_host64(t) for t in got]


def test_noalloc_matches_attn_bwd_twice_second_smaller(device):
    big = si.Workload("noalloc_big", 2, 6, 1000, 64, "bf16", 1.0, 1.0, 0.1, True)
    small = si.Workload("noalloc_small", 1, 3, 257, 64, "bf16", 1.0, 1.0, 0.1, True)
    print("\n[noalloc] B=2 H=6 S=1000 D=64 bf16, then B=1 H=3 S=257", flush=True)
    g1 = run_pair(big, device, seed=71)
    g2 = run_pair(small, device, seed=72)
    assert all(np.isfinite(a).all() for a in g1 + g2)


@pytest.mark.parametrize("w", [
    si.Workload("noalloc_f16_d128", 1, 4, 513, 128, "f16", 1.0, 1.0, 0.1, True),
    si.Workload("noalloc_f32_dense", 1, 2, 130, 64, "f32", 1.0, 1.0, 1.0, False),
], ids=lambda w: w.name)
def test_noalloc_other_types(device, w):
    print(f"\n[noalloc] {w.name}", flush=True)
    run_pair(w, device, seed=73)
