"""The fwd + bwd step captured into a HIP graph and replayed: every replay, with other
work and synchronizations between the replays, must reproduce the eagerly launched
step bit for bit (the kernels are deterministic and none of the captured entry points
records a memset or allocates).  Covers attn_fwd + attn_bwd and attn_fwd +
attn_bwd_noalloc, the entry point meant for callers that capture."""
import numpy as np
import pytest

import seeded_inputs as si
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    return gu.require_gpu()


def bits(t):
    torch = gu.torch_mod()
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("noalloc", [False, True], ids=["attn_bwd", "attn_bwd_noalloc"])
@pytest.mark.parametrize("w", [
    si.Workload("graph_bf16", 2, 4, 777, 64, "bf16", 1.0, 1.0, 0.1, True),
    si.Workload("graph_f16_d128", 1, 3, 300, 128, "f16", 1.0, 1.0, 0.1, True),
], ids=lambda w: w.name)
def test_graph_replays_equal_eager(device, w, noalloc):
    from causal_attention_flash_amd import _binding as bd
    torch = gu.torch_mod()
    print(f"\n[graph] {w.name} B={w.B} H={w.H} S={w.S} D={w.D} {w.dtype} noalloc={noalloc}", flush=True)
    x = si.make_inputs(w, seed=91)
    q, k, v, do = (gu.to_device(x, n, w.dtype, device) for n in ("q", "k", "v", "do"))
    B, H, S, D = q.shape
    dt = {"bf16": bd.ATTN_BF16, "f16": bd.ATTN_F16}[w.dtype]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=device)
    grads = [torch.empty_like(q) for _ in range(3)]
    nws = bd.c_attn_bwd_workspace_bytes(B, H, S, D, dt)
    ws = torch.empty(nws, dtype=torch.uint8, device=device)

    def step(stream):
        st = bd.c_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, S, D,
                           w.scale, int(w.causal), dt, stream)
        assert st == 0, bd.status_string(st)
        if noalloc:
            st = bd.c_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                       lse.data_ptr(), *(t.data_ptr() for t in grads), B, H, S, D, w.scale,
                                       int(w.causal), dt, stream)
        else:
            st = bd.c_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), *(t.data_ptr() for t in grads), ws.data_ptr(), nws, B, H, S, D,
                               w.scale, int(w.causal), dt, stream)
        assert st == 0, bd.status_string(st)

    cs = torch.cuda.current_stream(device)
    step(cs.cuda_stream)
    torch.cuda.synchronize()
    ref = [bits(t).clone() for t in [o, lse] + grads]

    side = torch.cuda.Stream(device)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in [o, lse] + grads:
            t.fill_(float("nan"))  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), [o, lse] + grads, ref):
            assert torch.equal(bits(a), b), (rep, name)
    assert np.isfinite(gu.to_host64(grads[0])).all()
