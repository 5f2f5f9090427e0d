"""GPU parity of the causal prefill path (tq_attend_prefill, through the C
ABI) against the CPU oracle's attend_prefill on the same seeded inputs.

The cache is encoded on the GPU and the oracle attends over the GPU's own
planes (codes, norms, QJL sign bits and residual norms) (encode parity is covered by the decode tests), so the comparison
isolates the attention kernel: max row-relative error <= 2e-3."""

import numpy as np
import pytest

import oracle as o
import seeded_inputs as si
from gpu_helpers import TOL, config_of, gpu_encode, log, rel_err, to_device, torch_cuda

pytestmark = pytest.mark.gpu

CASES = {
    # name: (small_workload kwargs, n_q)
    "d128_k3v4_g4_ragged": (dict(B=2, Hq=8, Hkv=2, N=700, bits_k=3, bits_v=4, wid=140), 150),
    "d128_k4v4_g1_f32": (dict(B=1, Hq=2, Hkv=2, N=333, bits_k=4, bits_v=4, norm_dtype="f32",
                              in_dtype="f32", wid=141), 70),
    "d128_k2v3_g3": (dict(B=1, Hq=6, Hkv=2, N=260, bits_k=2, bits_v=3, wid=142), 33),
    "d256_k2v2_g4": (dict(B=1, Hq=8, Hkv=2, d=256, N=300, bits_k=2, bits_v=2, wid=143), 100),
    "d256_k3v4_g2_f16in": (dict(B=1, Hq=4, Hkv=2, d=256, N=190, bits_k=3, bits_v=4,
                                in_dtype="f16", wid=144), 64),
    "d128_k3v4_g8_whole": (dict(B=1, Hq=8, Hkv=1, N=200, bits_k=3, bits_v=4, wid=145), 200),
    "d128_k3v4_sphere": (dict(B=1, Hq=8, Hkv=2, N=400, bits_k=3, bits_v=4, codebook="sphere",
                              wid=149), 90),
    # QJL: the sign dot is a second score product (one row block per wave;
    # d 256 runs with one tile buffer)
    "d128_k3qjl_v4_g4": (dict(B=2, Hq=8, Hkv=2, N=600, bits_k=3, bits_v=4, qjl=True, wid=150),
                         130),
    "d256_k3qjl_v4_g2": (dict(B=1, Hq=4, Hkv=2, d=256, N=330, bits_k=3, bits_v=4, qjl=True,
                              wid=151), 75),
    "d128_k2qjl_v2_g1_sphere": (dict(B=1, Hq=2, Hkv=2, N=250, bits_k=2, bits_v=2, qjl=True,
                                     codebook="sphere", wid=152), 40),
}


def _planes(cache, n, qjl=False):
    p = {k: getattr(cache, k)[:, :, :n].cpu().numpy() for k in ("kc", "vc")} | {
        k: getattr(cache, k)[:, :, :n].float().cpu().numpy().astype(np.float64)
        for k in ("kn", "vn")}
    if qjl:
        p["kq"] = cache.kq[:, :, :n].cpu().numpy()
        p["kr"] = cache.kr[:, :, :n].float().cpu().numpy().astype(np.float64)
    return p


def _run(w, n_q, scale=0.0):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    log(f"prefill case wid={w.wid} B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} N={w.N} n_q={n_q} "
        f"K{w.bits_k}/V{w.bits_v} qjl={w.qjl} norm={w.norm_dtype} in={w.in_dtype} "
        f"codebook={w.codebook}")
    cfg, cache = gpu_encode(w)
    raw, f32 = si.chunk_queries(w, n_q)
    q = to_device(raw, w.in_dtype)
    out = torch.empty((w.B, w.Hq, n_q, w.d), dtype=torch.float32, device="cuda")
    tq.tq_attend_prefill(cfg, q, cache, w.N, out, scale=scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = o.attend_prefill(f32.astype(np.float64), _planes(cache, w.N, w.qjl), w.N, d=w.d,
                           seed=w.seed, bits_k=w.bits_k, bits_v=w.bits_v, Hkv=w.Hkv,
                           scale=scale or None, qjl=w.qjl, qjl_seed=w.qjl_seed,
                           sphere=w.codebook == "sphere")
    err, abs_err = rel_err(got, ref)
    log(f"  max row-relative error {err:.2e} (abs {abs_err:.2e})")
    assert err <= TOL
    return cfg, cache, q, got


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_matches_oracle(name):
    kw, n_q = CASES[name]
    _run(si.small_workload(**kw), n_q)


def test_prefill_explicit_scale_and_one_query_equals_decode():
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(B=1, Hq=8, Hkv=2, N=500, bits_k=3, bits_v=4, wid=146)
    cfg, cache, q, got = _run(w, 1, scale=0.21)
    # a one-query chunk is the decode step of its last position
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))
    tq.tq_attend_decode(cfg, q[:, :, 0].contiguous(), cache, w.N, out, ws, scale=0.21)
    torch.cuda.synchronize()
    err, _ = rel_err(got[:, :, 0], out.cpu().numpy().astype(np.float64))
    assert err <= TOL


def test_prefill_rejects_bad_chunks():
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    q = torch.zeros((1, 4, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, 4, 8, 128), dtype=torch.float32, device="cuda")
    w2 = si.small_workload(B=1, Hq=4, Hkv=2, N=64, bits_k=3, bits_v=4, wid=148)
    cfg2, cache2 = gpu_encode(w2)
    with pytest.raises(tq.TqError) as e:
        tq.tq_attend_prefill(cfg2, q, cache2, 7, out)       # n_q > n_ctx
    assert e.value.status == tq.TQ_ERR_ARG
    with pytest.raises(tq.TqError) as e:
        tq.tq_attend_prefill(cfg2, q, cache2, 65, out)      # beyond capacity
    assert e.value.status == tq.TQ_ERR_CAPACITY


def test_prefill_context_shorter_than_capacity():
    # the cache has room for more tokens than the context holds: rows past
    # n_ctx (never written) must not be read
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(B=1, Hq=8, Hkv=2, N=300, bits_k=3, bits_v=4, wid=153)
    log(f"prefill with capacity 1000 > n_ctx {w.N}")
    cfg, cache = gpu_encode(w, capacity=1000)
    for name in ("kc", "vc", "kn", "vn"):                  # garbage past the context
        getattr(cache, name)[:, :, w.N:].fill_(0x7b if name in ("kc", "vc") else 1e4)
    n_q = 50
    raw, f32 = si.chunk_queries(w, n_q)
    out = torch.empty((w.B, w.Hq, n_q, w.d), dtype=torch.float32, device="cuda")
    tq.tq_attend_prefill(cfg, to_device(raw, w.in_dtype), cache, w.N, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = o.attend_prefill(f32.astype(np.float64), _planes(cache, w.N), w.N, d=w.d, seed=w.seed,
                           bits_k=w.bits_k, bits_v=w.bits_v, Hkv=w.Hkv)
    err, _ = rel_err(got, ref)
    log(f"  max row-relative error {err:.2e}")
    assert err <= TOL
