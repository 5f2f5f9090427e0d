"""Parity of the group-affine variant (rotated keys, group 64, fp16 scale and
bias) on the GPU against the oracle in oracle/affine.py.

Encode: value codes, scales and biases bit-exact on every row; key rows
bit-exact outside the oracle's decision band (a code within 1e-9 of a
rounding tie, or a scale or bias within 1e-9 of an fp16 rounding boundary,
where the rotation's summation order can decide). Decode: the oracle's attention over
its own cache (never the GPU's), within TOL row-relative."""

import numpy as np
import pytest

import oracle as o
import seeded_inputs as si
from gpu_helpers import TOL, kv_host, log, rel_err, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def _cfg(w):
    import decode_attention_seeded_amd as tq
    return tq.AffineConfig(d=w.d, bits_k=w.bits_k, bits_v=w.bits_v, group=64, seed=w.seed)


def _gpu_encode(w, capacity=None, chunks=None):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    cfg = _cfg(w)
    cache = tq.AffineCache(cfg, w.B, w.Hkv, capacity or w.N)
    spans = chunks or [(0, w.N)]
    for t0, t1 in spans:
        rk, rv, _, _ = kv_host(w, t0, t1)
        tq.tq_affine_encode_kv(cfg, to_device(rk, w.in_dtype), to_device(rv, w.in_dtype), t0,
                               cache)
    torch.cuda.synchronize()
    return cfg, cache


def _oracle_cache(w, n=None):
    _, _, fk, fv = kv_host(w, 0, n or w.N)
    return o.affine_encode_kv(fk, fv, bits_k=w.bits_k, bits_v=w.bits_v, seed=w.seed), fk, fv


def _compare_encode(w, cache, ref, fv, n):
    # keys: the two sides rotate with different (equally exact) summation
    # orders, so rows in the decision band may differ. Values are not
    # rotated: every step from the (exactly representable) inputs is one
    # correctly rounded fp64 operation on both sides, so every value row,
    # exact ties included, must match.
    # (At d = 256 with 16-bit inputs the rotated keys are exact in fp64 on
    # both sides, so exact ties land in the band but still agree.)
    ky = ref["ky"]
    bad_k = o.affine_code_ambiguous(ky, w.bits_k)
    bad_v = np.zeros(bad_k.shape, dtype=bool)
    assert bad_k.mean() < 0.05
    got = {name: getattr(cache, name)[:, :, :n].cpu().numpy()
           for name in ("kc", "vc", "ks", "kb", "vs", "vb")}
    differ = 0
    for name, bad in (("kc", bad_k), ("ks", bad_k), ("kb", bad_k),
                      ("vc", bad_v), ("vs", bad_v), ("vb", bad_v)):
        want = ref[name]
        g = got[name].view(np.uint16) if got[name].dtype == np.float16 else got[name]
        r = want.view(np.uint16) if want.dtype == np.float16 else want
        rows = np.any(g != r, axis=-1)
        assert not np.any(rows & ~bad), f"{name}: {int((rows & ~bad).sum())} rows differ off the band"
        differ += int(rows.sum())
    log(f"encode parity: {int(bad_k.sum())} key rows in the band, {differ} plane rows differ there")


def _decode(w, cfg, cache, n_ctx, splits=0, scale=0.0):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    qraw, qf = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_affine_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, n_ctx, splits))
    tq.tq_affine_attend_decode(cfg, q, cache, n_ctx, out, ws, scale=scale, splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), np.asarray(qf, np.float64)


CASES = {
    "d128_k4v4_gqa": dict(B=1, Hq=8, Hkv=2, d=128, N=1000, bits_k=4, bits_v=4),
    "d128_k3v3_ragged_g3": dict(B=2, Hq=6, Hkv=2, d=128, N=777, bits_k=3, bits_v=3,
                                in_dtype="f32"),
    "d128_k2v4_g1": dict(B=1, Hq=3, Hkv=3, d=128, N=300, bits_k=2, bits_v=4,
                         in_dtype="f16"),
    "d256_k4v2_outlier": dict(B=1, Hq=4, Hkv=1, d=256, N=650, bits_k=4, bits_v=2,
                              structure="outlier"),
    "d256_k3v4_g2": dict(B=2, Hq=4, Hkv=2, d=256, N=129, bits_k=3, bits_v=4, seed=7),
    # the matrix-core kernel (4-bit keys and values, d 128) at one and two
    # query heads per workgroup
    "d128_k4v4_g1_f16in": dict(B=2, Hq=2, Hkv=2, d=128, N=900, bits_k=4, bits_v=4,
                               in_dtype="f16"),
    "d128_k4v4_g2_ragged": dict(B=1, Hq=4, Hkv=2, d=128, N=1531, bits_k=4, bits_v=4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_affine_encode_and_decode_match_oracle(name):
    kw = CASES[name]
    w = si.small_workload(wid=300 + sorted(CASES).index(name), **kw)
    log(f"affine case {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} N={w.N} "
        f"K{w.bits_k}V{w.bits_v} {w.in_dtype} {w.structure}")
    cfg, cache = _gpu_encode(w)
    ref, _, fv = _oracle_cache(w)
    _compare_encode(w, cache, ref, fv, w.N)
    for n_ctx, splits in ((w.N, 0), (w.N, 1), (max(1, w.N // 3), 0), (1, 0)):
        got, qf = _decode(w, cfg, cache, n_ctx, splits)
        want = o.affine_attend(qf, {k: ref[k] for k in ("kc", "vc", "ks", "kb", "vs", "vb")},
                               n_ctx, d=w.d, seed=w.seed, bits_k=w.bits_k, bits_v=w.bits_v,
                               Hkv=w.Hkv)
        err, abs_err = rel_err(got, want)
        log(f"  n_ctx={n_ctx} splits={splits}: row-relative {err:.2e} (abs {abs_err:.2e})")
        assert np.all(np.isfinite(got))
        assert err <= TOL


def test_affine_chunked_append_equals_bulk():
    w = si.small_workload(wid=320, B=1, Hq=4, Hkv=2, d=128, N=500, bits_k=4, bits_v=4)
    log("affine chunked append: N=500 in chunks 0-200, 200-201, 201-500, capacity 600")
    _, bulk = _gpu_encode(w, capacity=600)
    _, chunked = _gpu_encode(w, capacity=600, chunks=[(0, 200), (200, 201), (201, 500)])
    for name in ("kc", "vc", "ks", "kb", "vs", "vb"):
        a = getattr(bulk, name)[:, :, :500].cpu().numpy()
        b = getattr(chunked, name)[:, :, :500].cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name


def test_affine_long_context_sampled_heads():
    # the scale of the long-context workload on one batch row: 8 KV heads,
    # 32 query heads, 131072 tokens, K4/V4 (the README's iso-byte 4-bit
    # format); the oracle runs on every head
    w = si.small_workload(wid=330, B=1, Hq=32, Hkv=8, d=128, N=131072, bits_k=4, bits_v=4)
    log("affine long context: B=1 Hq=32 Hkv=8 d=128 N=131072 K4V4")
    cfg, cache = _gpu_encode(w)
    ref, _, fv = _oracle_cache(w)
    _compare_encode(w, cache, ref, fv, w.N)
    got, qf = _decode(w, cfg, cache, w.N)
    want = o.affine_attend(qf, {k: ref[k] for k in ("kc", "vc", "ks", "kb", "vs", "vb")},
                           w.N, d=w.d, seed=w.seed, bits_k=4, bits_v=4, Hkv=w.Hkv)
    err, abs_err = rel_err(got, want)
    log(f"  row-relative {err:.2e} (abs {abs_err:.2e})")
    assert err <= TOL


def test_affine_explicit_scale_and_split_counts():
    # an explicit softmax scale, and requested split counts from 1 to far
    # more than the context has tiles (the library clamps them); every
    # result against the oracle and all split counts against each other
    w = si.small_workload(wid=340, B=1, Hq=8, Hkv=4, d=128, N=2000, bits_k=4, bits_v=3)
    log("affine scale/splits: B=1 Hq=8 Hkv=4 d=128 N=2000 K4V3, scale 0.2, splits 1..5000")
    cfg, cache = _gpu_encode(w)
    ref, _, _ = _oracle_cache(w)
    planes = {k: ref[k] for k in ("kc", "vc", "ks", "kb", "vs", "vb")}
    outs = []
    for splits in (1, 3, 8, 5000):
        got, qf = _decode(w, cfg, cache, w.N, splits=splits, scale=0.2)
        want = o.affine_attend(qf, planes, w.N, d=w.d, seed=w.seed, bits_k=4, bits_v=3,
                               Hkv=w.Hkv, scale=0.2)
        err, _ = rel_err(got, want)
        log(f"  splits={splits}: row-relative {err:.2e}")
        assert err <= TOL
        outs.append(got)
    for g in outs[1:]:
        assert rel_err(g, outs[0])[0] < 1e-5


def test_affine_k4v4_split_counts_and_valu_kernel(monkeypatch):
    # 4-bit keys and values run on the matrix cores: requested split counts
    # against the oracle, and the VALU kernel (TQ_DECODE_VALU=1) on the same
    # cache against the oracle and the matrix-core result
    w = si.small_workload(wid=350, B=1, Hq=8, Hkv=2, d=128, N=3000, bits_k=4, bits_v=4)
    log("affine K4V4: B=1 Hq=8 Hkv=2 d=128 N=3000, splits 1/3/8, and the VALU kernel")
    cfg, cache = _gpu_encode(w)
    ref, _, _ = _oracle_cache(w)
    planes = {k: ref[k] for k in ("kc", "vc", "ks", "kb", "vs", "vb")}
    want = None
    outs = []
    for splits in (1, 3, 8):
        got, qf = _decode(w, cfg, cache, w.N, splits=splits)
        if want is None:
            want = o.affine_attend(qf, planes, w.N, d=w.d, seed=w.seed, bits_k=4, bits_v=4,
                                   Hkv=w.Hkv)
        err, _ = rel_err(got, want)
        log(f"  matrix cores, splits={splits}: row-relative {err:.2e}")
        assert err <= TOL
        outs.append(got)
    monkeypatch.setenv("TQ_DECODE_VALU", "1")
    got, _ = _decode(w, cfg, cache, w.N)
    err, _ = rel_err(got, want)
    log(f"  VALU kernel: row-relative {err:.2e}; vs matrix cores {rel_err(got, outs[0])[0]:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("vs,qs", [(300.0, 1.0), (1e-3, 1.0), (1e4, 1.0), (1.0, 3.0),
                                   (1.0, 1e-5)])
def test_affine_k4v4_far_from_unit_scale(vs, qs):
    # the matrix-core kernel's fp16 operands (query with its power-of-two
    # scale, weights times the value scale with their band, codes as 64 + c)
    # on values and queries far from unit scale; fp32 inputs so that both
    # sides see the same scaled numbers
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(wid=360, B=1, Hq=8, Hkv=2, d=128, N=1300, bits_k=4, bits_v=4,
                          in_dtype="f32")
    log(f"affine K4V4 range: values x{vs:g}, queries x{qs:g}")
    _, _, fk, fv = kv_host(w, 0, w.N)
    fv = fv * vs
    qf = si.queries(w)[1].astype(np.float64) * qs
    cfg = _cfg(w)
    cache = tq.AffineCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_affine_encode_kv(cfg, torch.from_numpy(fk.astype(np.float32)).cuda(),
                           torch.from_numpy(fv.astype(np.float32)).cuda(), 0, cache)
    q = torch.from_numpy(qf.astype(np.float32)).cuda()
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_affine_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))
    tq.tq_affine_attend_decode(cfg, q, cache, w.N, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = o.affine_encode_kv(fk, fv, bits_k=4, bits_v=4, seed=w.seed)
    want = o.affine_attend(qf.astype(np.float32).astype(np.float64),
                           {k: ref[k] for k in ("kc", "vc", "ks", "kb", "vs", "vb")}, w.N,
                           d=w.d, seed=w.seed, bits_k=4, bits_v=4, Hkv=w.Hkv)
    err, abs_err = rel_err(got, want)
    log(f"  row-relative {err:.2e} (abs {abs_err:.2e})")
    assert np.isfinite(got).all()
    assert err <= TOL
