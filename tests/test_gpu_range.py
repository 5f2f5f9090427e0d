"""Input range of the decode and prefill kernels: values scaled far up or
down (value norms 300x, 1e5x larger or 1e3x, 1e6x smaller than unit-variance
rows) and queries scaled by 3, 1e-5, 1e3 or 1e6, against the oracle on the
same scaled inputs. The kernels multiply fp16 operands (the rotated query,
the softmax weight times the value norm); both are kept inside fp16's range
by powers of two that are undone in fp32, so no scale overflows or flushes
to zero.

Values at any scale, and queries x1e-5, keep the usual 2e-3 bar. The query
itself is rounded to fp16 (relative 2^-11 per element), so a score's error,
and with it the output's, grows in proportion to |q| |k|: measured against
the oracle, the decode's error is 4.3e-4 at x1, 2.4e-3 at x10 and 9.7e-3 at
x100, the prefill's 6-7e-4 at x1, 1.5-2.6e-3 at x3 and 4-7e-3 at x10 (over
four seeds each). Queries x3 are therefore held to 2e-3 times the query
scale. For queries x1e3 (rows with near-ties between top tokens) and x1e6
(whose rotated elements pass fp16's largest value unless scaled) the check
is the property that holds at any temperature: a finite output inside the
per-coordinate range of the dequantized value rows (a convex combination of
them).

Value norms that change along the context (a ramp over 2^20, a sawtooth of
2^+-8) make the kernels move their per-tile power of two for the value
scales, and rescale the accumulators, many times within one call; those
cases keep the 2e-3 bar.

Inputs are fp32 (so the scaled values reach both sides unrounded); norms are
fp16 where they fit its range and fp32 for the 1e5 and 1e-6 cases."""

import numpy as np
import pytest

import oracle as o
import seeded_inputs as si
from gpu_helpers import TOL, config_of, log, rel_err, to_device, torch_cuda

pytestmark = pytest.mark.gpu

FORMATS = {
    # name: small_workload kwargs (the decode kernel each format runs)
    "k3v4": dict(B=1, Hq=8, Hkv=2, N=1500, bits_k=3, bits_v=4),
    "d256_k2v2": dict(B=1, Hq=4, Hkv=1, d=256, N=1100, bits_k=2, bits_v=2),
    "k3qjl_v4": dict(B=1, Hq=8, Hkv=2, N=1200, bits_k=3, bits_v=4, qjl=True),
    "k3v3": dict(B=1, Hq=6, Hkv=2, N=900, bits_k=3, bits_v=3),
}
SCALES = {
    # name: (value scale, query scale, norm dtype)
    "v300": (300.0, 1.0, "f16"),
    "v1e-3": (1e-3, 1.0, "f16"),
    "v1e5": (1e5, 1.0, "f32"),
    "v1e-6": (1e-6, 1.0, "f32"),
    "q3": (1.0, 3.0, "f16"),
    "q1e3": (1.0, 1e3, "f16"),
    "q1e6": (1.0, 1e6, "f16"),
    "q1e-5": (1.0, 1e-5, "f16"),
}


def _scaled_inputs(w, vs, qs, n_q=0):
    """K, V [B][Hkv][N][d] and q ([B][Hq][d], or a prefill chunk) as fp32,
    the values and queries multiplied by vs and qs."""
    ks, vv = [], []
    for b in range(w.B):
        for h in range(w.Hkv):
            ks.append(si.kv_rows(w, si.T_K, b, h, 0, w.N)[1])
            vv.append(si.kv_rows(w, si.T_V, b, h, 0, w.N)[1] * np.float32(vs))
    shp = (w.B, w.Hkv, w.N, w.d)
    k = np.stack(ks).reshape(shp).astype(np.float32)
    v = np.stack(vv).reshape(shp).astype(np.float32)
    q = (si.chunk_queries(w, n_q)[1] if n_q else si.queries(w)[1]) * np.float32(qs)
    return k, v, q.astype(np.float32)


def _check(got, want, ref, w, scl):
    assert np.isfinite(got).all(), "non-finite output"
    if scl not in ("q1e3", "q1e6"):
        err, abs_err = rel_err(got, want)
        tol = TOL * max(1.0, SCALES[scl][1])      # fp16 query rounding scales with |q|
        log(f"  max row-relative error {err:.2e} (abs {abs_err:.2e}), bar {tol:.1e}")
        assert err <= tol
        return
    # per KV head: every output coordinate within [min, max] of the
    # dequantized value rows (original frame) over the context
    for b in range(w.B):
        for h in range(w.Hkv):
            vc = o.unpack_codes(ref["vc"][b, h], w.bits_v, w.d)
            vhat = o.rht_inverse(o.dequant_rot(vc, ref["vn"][b, h], w.bits_v), w.seed)
            lo, hi = vhat.min(axis=0), vhat.max(axis=0)
            pad = 1e-3 * (hi - lo)
            g = got[b, h * w.G:(h + 1) * w.G].reshape(-1, w.d)
            assert (g >= lo - pad).all() and (g <= hi + pad).all(), "outside the value hull"
    log("  finite and inside the value rows' coordinate range")


def _case(fmt, scl, wid):
    vs, qs, nd = SCALES[scl]
    return si.small_workload(wid=wid, in_dtype="f32", norm_dtype=nd, **FORMATS[fmt]), vs, qs


@pytest.mark.parametrize("scl", sorted(SCALES))
@pytest.mark.parametrize("fmt", sorted(FORMATS))
def test_decode_far_from_unit_scale(fmt, scl):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w, vs, qs = _case(fmt, scl, 200 + sorted(FORMATS).index(fmt))
    log(f"decode {fmt} with values x{vs:g}, queries x{qs:g} ({w.norm_dtype} norms)")
    k, v, q = _scaled_inputs(w, vs, qs)
    cfg = config_of(w)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_encode_kv(cfg, to_device(k, "f32"), to_device(v, "f32"), 0, cache)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))
    tq.tq_attend_decode(cfg, to_device(q, "f32"), cache, w.N, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = o.encode_kv(k.astype(np.float64), v.astype(np.float64), seed=w.seed, bits_k=w.bits_k,
                      bits_v=w.bits_v, norm_dtype=w.norm_dtype, qjl=w.qjl, qjl_seed=w.qjl_seed)
    want = o.attend(q.astype(np.float64), ref, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k,
                    bits_v=w.bits_v, Hkv=w.Hkv, qjl=w.qjl, qjl_seed=w.qjl_seed)
    _check(got, want, ref, w, scl)


@pytest.mark.parametrize("scl", sorted(SCALES))
@pytest.mark.parametrize("fmt", ["k3v4", "k3qjl_v4"])
def test_prefill_far_from_unit_scale(fmt, scl):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w, vs, qs = _case(fmt, scl, 210 + (fmt == "k3qjl_v4"))
    n_q = 130
    log(f"prefill {fmt} with values x{vs:g}, queries x{qs:g} ({w.norm_dtype} norms)")
    k, v, q = _scaled_inputs(w, vs, qs, n_q)
    cfg = config_of(w)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_encode_kv(cfg, to_device(k, "f32"), to_device(v, "f32"), 0, cache)
    out = torch.empty((w.B, w.Hq, n_q, w.d), dtype=torch.float32, device="cuda")
    tq.tq_attend_prefill(cfg, to_device(q, "f32"), cache, w.N, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = o.encode_kv(k.astype(np.float64), v.astype(np.float64), seed=w.seed, bits_k=w.bits_k,
                      bits_v=w.bits_v, norm_dtype=w.norm_dtype, qjl=w.qjl, qjl_seed=w.qjl_seed)
    want = o.attend_prefill(q.astype(np.float64), ref, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k,
                            bits_v=w.bits_v, Hkv=w.Hkv, qjl=w.qjl, qjl_seed=w.qjl_seed)
    _check(got, want, ref, w, scl)


# Value norms that change along the context: the kernels' per-tile power of
# two for the value scales has to move (a ramp over 2^20: many moves one
# way; a sawtooth of 2^+-8 with a 37-token period: tiles that mix both and
# moves both ways), with the accumulators rescaled on every move.
PROFILES = {
    "ramp": lambda t, n: np.exp2(-10.0 + 20.0 * t / max(n - 1, 1)),
    "saw": lambda t, n: np.where((t // 37) % 2 == 0, 2.0 ** 8, 2.0 ** -8),
}


def _profiled_inputs(w, prof, n_q=0):
    k, v, q = _scaled_inputs(w, 1.0, 1.0, n_q)
    f = PROFILES[prof](np.arange(w.N), w.N).astype(np.float32)
    return k, (v * f[None, None, :, None]).astype(np.float32), q


@pytest.mark.parametrize("prof", sorted(PROFILES))
@pytest.mark.parametrize("fmt", ["k3v4", "k3qjl_v4", "d256_k2v2"])
def test_decode_value_norms_along_the_context(fmt, prof):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(wid=230 + sorted(FORMATS).index(fmt), in_dtype="f32",
                          norm_dtype="f16", **FORMATS[fmt])
    log(f"decode {fmt} with value norms along a {prof} profile")
    k, v, q = _profiled_inputs(w, prof)
    cfg = config_of(w)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_encode_kv(cfg, to_device(k, "f32"), to_device(v, "f32"), 0, cache)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N))
    tq.tq_attend_decode(cfg, to_device(q, "f32"), cache, w.N, out, ws)
    torch.cuda.synchronize()
    ref = o.encode_kv(k.astype(np.float64), v.astype(np.float64), seed=w.seed, bits_k=w.bits_k,
                      bits_v=w.bits_v, norm_dtype=w.norm_dtype, qjl=w.qjl, qjl_seed=w.qjl_seed)
    want = o.attend(q.astype(np.float64), ref, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k,
                    bits_v=w.bits_v, Hkv=w.Hkv, qjl=w.qjl, qjl_seed=w.qjl_seed)
    err, abs_err = rel_err(out.cpu().numpy().astype(np.float64), want)
    log(f"  max row-relative error {err:.2e} (abs {abs_err:.2e})")
    assert err <= TOL


@pytest.mark.parametrize("prof", sorted(PROFILES))
@pytest.mark.parametrize("fmt", ["k3v4", "k3qjl_v4"])
def test_prefill_value_norms_along_the_context(fmt, prof):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(wid=240 + (fmt == "k3qjl_v4"), in_dtype="f32", norm_dtype="f16",
                          **FORMATS[fmt])
    n_q = 130
    log(f"prefill {fmt} with value norms along a {prof} profile")
    k, v, q = _profiled_inputs(w, prof, n_q)
    cfg = config_of(w)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_encode_kv(cfg, to_device(k, "f32"), to_device(v, "f32"), 0, cache)
    out = torch.empty((w.B, w.Hq, n_q, w.d), dtype=torch.float32, device="cuda")
    tq.tq_attend_prefill(cfg, to_device(q, "f32"), cache, w.N, out)
    torch.cuda.synchronize()
    ref = o.encode_kv(k.astype(np.float64), v.astype(np.float64), seed=w.seed, bits_k=w.bits_k,
                      bits_v=w.bits_v, norm_dtype=w.norm_dtype, qjl=w.qjl, qjl_seed=w.qjl_seed)
    want = o.attend_prefill(q.astype(np.float64), ref, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k,
                            bits_v=w.bits_v, Hkv=w.Hkv, qjl=w.qjl, qjl_seed=w.qjl_seed)
    err, abs_err = rel_err(out.cpu().numpy().astype(np.float64), want)
    log(f"  max row-relative error {err:.2e} (abs {abs_err:.2e})")
    assert err <= TOL
