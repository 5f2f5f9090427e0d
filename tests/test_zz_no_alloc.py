"""The allocation-free decode entry point (tq_attend_decode_noalloc, static
per-GPU scratch buffer) against tq_attend_decode on a caller workspace: two
calls in a row, the second smaller, through the C ABI; the same kernels run,
so the outputs must be equal bit for bit. Also the host-side rejection of a
call that needs more scratch than the buffer holds."""

import numpy as np
import pytest

import seeded_inputs as si
from gpu_helpers import config_of, gpu_encode, log, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def _both(w, cfg, cache, q, n_ctx, splits=0):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    want = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, n_ctx, splits))
    tq.tq_attend_decode(cfg, q, cache, n_ctx, want, ws, splits=splits)
    got = torch.full_like(want, float("nan"))
    tq.tq_attend_decode_noalloc(cfg, q, cache, n_ctx, got, splits=splits)
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("bits_v,qjl", [(4, False), (2, False), (4, True), (3, False)])
def test_noalloc_equals_workspace_decode_twice(bits_v, qjl):
    torch = torch_cuda()
    w = si.small_workload(B=2, Hq=8, Hkv=2, N=5000, bits_k=3, bits_v=bits_v, qjl=qjl,
                          wid=170 + bits_v + 10 * qjl)
    log(f"no-alloc decode: K3/V{bits_v} qjl={qjl}")
    cfg, cache = gpu_encode(w)
    qraw, _ = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    got, want = _both(w, cfg, cache, q, w.N)
    assert np.isfinite(got.cpu().numpy()).all()
    assert torch.equal(got, want)
    # second call, smaller: fewer tokens and an explicit split count
    got, want = _both(w, cfg, cache, q, 1777, splits=3)
    assert np.isfinite(got.cpu().numpy()).all()
    assert torch.equal(got, want)
    # and a smaller batch on a cache of its own
    w1 = si.small_workload(B=1, Hq=4, Hkv=1, N=700, bits_k=3, bits_v=bits_v, qjl=qjl,
                           wid=180 + bits_v + 10 * qjl)
    cfg1, cache1 = gpu_encode(w1)
    q1 = to_device(si.queries(w1)[0], w1.in_dtype)
    got, want = _both(w1, cfg1, cache1, q1, w1.N)
    assert torch.equal(got, want)


def test_noalloc_rejects_calls_beyond_its_scratch():
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    # 64 x 32 query heads, d 256, 4 splits: the partials alone take
    # 2048 * 4 * 258 * 4 bytes > 8 MiB; the check runs on the host, before any
    # HIP call, so the cache's bytes are never read
    w = si.small_workload(B=64, Hq=32, Hkv=8, d=256, N=2048, wid=190)
    cfg = config_of(w)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    q = torch.zeros((w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    need = tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N, 4)
    assert need > 8 << 20
    with pytest.raises(tq.TqError) as e:
        tq.tq_attend_decode_noalloc(cfg, q, cache, w.N, out, splits=4)
    assert e.value.status == tq.TQ_ERR_WORKSPACE
