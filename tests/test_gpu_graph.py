"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph), as
bench.py times it: append encode + decode (as two calls, or as the one
tq_append_chunk_attend_decode call), replayed several times with eager
calls and synchronizations between the replays. Every replay's output and
cache bytes must equal the eager step's bit for bit; this also exercises the
decode's arrival counters, which every call leaves at zero."""

import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import config_of, kv_host, log, to_device, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("bits_v,qjl", [(4, False), (2, False), (4, True), (3, False)])
def test_graph_replays_equal_eager_step(bits_v, qjl, fused):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(B=2, Hq=8, Hkv=2, N=3000, bits_k=3, bits_v=bits_v, wid=150 + bits_v,
                          qjl=qjl)
    log(f"graph replay: K3/V{bits_v} qjl={qjl} fused={fused}")
    cfg = config_of(w)
    rk, rv, _, _ = kv_host(w, 0, w.N)
    K, V = to_device(rk, w.in_dtype), to_device(rv, w.in_dtype)
    A = 256
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_encode_kv(cfg, K[:, :, :w.N - A].contiguous(), V[:, :, :w.N - A].contiguous(), 0, cache)
    k_app, v_app = K[:, :, w.N - A:].contiguous(), V[:, :, w.N - A:].contiguous()
    qraw, _ = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))

    def step():
        if fused:
            tq.tq_append_chunk_attend_decode(cfg, k_app, v_app, q, cache, w.N, out, ws)
        else:
            tq.tq_encode_kv(cfg, k_app, v_app, w.N - A, cache)
            tq.tq_attend_decode(cfg, q, cache, w.N, out, ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    planes = [cache.kc.clone(), cache.vc.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    ws2 = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, 1700))
    for r in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager step"
        assert torch.equal(cache.kc, planes[0]) and torch.equal(cache.vc, planes[1])
        # eager work between replays: a shorter decode on another workspace
        tq.tq_attend_decode(cfg, q, cache, 1700, other, ws2)
        torch.cuda.synchronize()
        assert np.isfinite(other.cpu().numpy()).all()
    # and the eager step once more on the graph's workspace
    out.fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    assert torch.equal(out, eager)
