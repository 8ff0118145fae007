"""Shared helpers for the GPU parity tests: device transfer, comparisons, tolerances.

Tolerances (written here, applied per output tensor):
* bf16 inputs: max |gpu - oracle| <= 2e-2 for O, LSE, dQ, dK, dV;
* fp16 inputs: max |gpu - oracle| <= 5e-3 for the same outputs.  Derivation: the
  error terms are the 16-bit roundings of the outputs, of P and dS before the
  MFMAs and of O where delta is formed; binary16 carries 3 more fraction bits
  than bfloat16, so each shrinks by 2^-3 against the bf16 case (2e-2 -> 2.5e-3),
  and the output rounding alone reaches 2^-9 ~ 2e-3 for |x| in [4, 8), which
  the long workload's O attains; 5e-3 covers both with a factor of ~2;
* fp32 inputs: max |gpu - oracle| / max |oracle| <= 1e-4 per tensor (the relative
  error is taken against the tensor's largest magnitude because dQ's first row
  is exactly zero, where an elementwise relative error is undefined); a tensor
  whose reference is identically zero is held to max |gpu| <= 1e-4.
"""
import numpy as np

BF16_ABS_TOL = 2e-2
F16_ABS_TOL = 5e-3
F32_REL_TOL = 1e-4
OUTPUTS = ("o", "lse", "dq", "dk", "dv")


def torch_mod():
    import torch
    return torch


def require_gpu():
    import pytest
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import causal_attention_flash_amd as caf
    caf.load_library()  # raises if the HIP library is missing: no fallback
    return torch.device("cuda:0")


def to_device(x: dict, name: str, dtype: str, device):
    torch = torch_mod()
    if dtype in ("bf16", "f16"):
        bits = np.ascontiguousarray(x[name + "_bits"]).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return torch.from_numpy(np.ascontiguousarray(x[name], dtype=np.float32)).to(device)


def to_host64(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().to(torch.float64).cpu().numpy()


def run_gpu(x: dict, w, device, causal=True, scale=None):
    """attn_fwd then attn_bwd (fed the forward's own O and LSE), synchronised; float64 numpy outputs."""
    import causal_attention_flash_amd as caf
    torch = torch_mod()
    scale = w.scale if scale is None else scale
    q, k, v, do = (to_device(x, n, w.dtype, device) for n in ("q", "k", "v", "do"))
    o, lse = caf.attn_fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = caf.attn_bwd(q, k, v, o, do, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return {"o": to_host64(o), "lse": to_host64(lse), "dq": to_host64(dq), "dk": to_host64(dk),
            "dv": to_host64(dv)}


def errors(gpu: dict, ref: dict, heads=None) -> dict:
    """Per output: (max abs error, max |ref|) over the given (b, h) heads (all if None)."""
    out = {}
    for n in OUTPUTS:
        g, r = gpu[n], ref[n]
        if heads is not None:
            g = np.stack([g[b, h] for b, h in heads])
            r = np.stack([r[b, h] for b, h in heads]) if r.ndim == gpu[n].ndim else r
        assert np.isfinite(g).all(), f"{n}: non-finite GPU output"
        out[n] = (float(np.abs(g - r).max()), float(np.abs(r).max()))
    return out


def check(errs: dict, dtype: str, label: str = ""):
    lines = []
    bad = []
    for n, (e, mref) in errs.items():
        if dtype in ("bf16", "f16"):
            tol = BF16_ABS_TOL if dtype == "bf16" else F16_ABS_TOL
            ok = e <= tol
            lines.append(f"{n}: max|err| {e:.3e} (tol {tol}) max|ref| {mref:.3g}")
        else:
            # an identically zero reference (e.g. dQ, dK at S = 1) has no relative
            # error; there the bound is absolute, on the unit scale of the inputs
            rel = e / mref if mref > 0 else e
            ok = rel <= F32_REL_TOL
            lines.append(f"{n}: rel {rel:.3e} (tol {F32_REL_TOL}) max|ref| {mref:.3g}")
        if not ok:
            bad.append(n)
    msg = f"{label}\n" + "\n".join(lines)
    print(msg, flush=True)
    assert not bad, f"outside tolerance: {bad}\n{msg}"
