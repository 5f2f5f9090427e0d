"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
the same seeded inputs: small shapes that span several tiles plus a ragged
tail, every bit-width combination, GQA group sizes 1/2/3/4/8, d = 128/256,
QJL, fp32/fp16 norms, appends, explicit scale, split counts, edge cases.

Bars: packed codes, norms and QJL sign bits bit-exact except the counted
boundary cases; attention output max row-relative error <= 2e-3."""

import math

import numpy as np
import pytest

import oracle as o
import seeded_inputs as si
from gpu_helpers import (TOL, compare_codes, config_of, gpu_decode, gpu_encode, kv_host,
                         log, oracle_encode, rel_err, to_device, torch_cuda)

pytestmark = pytest.mark.gpu

SMALL = {
    # name: small_workload kwargs
    "d128_k4v4_f32norm_f32in_g1": dict(B=1, Hq=1, Hkv=1, N=700, bits_k=4, bits_v=4,
                                       norm_dtype="f32", in_dtype="f32", wid=101),
    "d128_k3v4_gqa4": dict(B=2, Hq=8, Hkv=2, N=1000, bits_k=3, bits_v=4, wid=102),
    "d256_k2v2_outlier": dict(B=2, Hq=4, Hkv=1, d=256, N=1100, bits_k=2, bits_v=2,
                              structure="outlier", wid=103),
    "d128_k3qjl_v4_corr": dict(B=2, Hq=8, Hkv=2, N=900, bits_k=3, bits_v=4, qjl=True,
                               structure="correlated", wid=104),
    "d128_k2v3_g2_f16in": dict(B=1, Hq=4, Hkv=2, N=513, bits_k=2, bits_v=3,
                               in_dtype="f16", wid=105),
    "d128_k4v2_g8": dict(B=1, Hq=8, Hkv=1, N=600, bits_k=4, bits_v=2, wid=106),
    "d128_k3v3_g3": dict(B=1, Hq=6, Hkv=2, N=450, bits_k=3, bits_v=3, wid=107),
    "d256_k3qjl_v4": dict(B=1, Hq=4, Hkv=2, d=256, N=1300, bits_k=3, bits_v=4, qjl=True,
                          structure="correlated", wid=108),
    "d256_k4v3_f32norm": dict(B=1, Hq=2, Hkv=1, d=256, N=520, bits_k=4, bits_v=3,
                              norm_dtype="f32", wid=109),
    "d128_n1": dict(B=2, Hq=4, Hkv=2, N=1, bits_k=3, bits_v=4, wid=110),
    # one query head per KV head with f32 norms: the score scaling follows the
    # last DPP dot of the K phase closely (dot-result wait states)
    "d128_k3v4_f32norm_g1": dict(B=2, Hq=2, Hkv=2, N=1500, bits_k=3, bits_v=4,
                                 norm_dtype="f32", wid=111),
    # matrix-core decode formats not covered above: d = 256 with 4-bit values
    # (two-dword value slices), 2-bit keys at d = 128, 4-bit keys at d = 256
    "d256_k3v4_g2": dict(B=1, Hq=4, Hkv=2, d=256, N=700, bits_k=3, bits_v=4, wid=112),
    "d256_k4v2_f32norm_g4": dict(B=1, Hq=4, Hkv=1, d=256, N=650, bits_k=4, bits_v=2,
                                 norm_dtype="f32", wid=113),
    "d128_k2v4_g4": dict(B=1, Hq=8, Hkv=2, N=800, bits_k=2, bits_v=4, wid=114),
    # the exact finite-d marginal codebook (encode thresholds, decode tables,
    # QJL residual centroids)
    "d128_k3v4_sphere": dict(B=1, Hq=8, Hkv=2, N=900, bits_k=3, bits_v=4, codebook="sphere",
                             wid=115),
    "d256_k2v2_sphere_qjl": dict(B=1, Hq=4, Hkv=2, d=256, N=520, bits_k=2, bits_v=2, qjl=True,
                                 codebook="sphere", wid=116),
    # 3-bit values on the matrix cores: windows of the column's 3 or 6 bytes
    # at every byte offset, with QJL, and d = 256 with 2-bit keys
    "d128_k3qjl_v3_g4": dict(B=2, Hq=8, Hkv=2, N=700, bits_k=3, bits_v=3, qjl=True,
                             structure="correlated", wid=117),
    "d256_k2v3_g4": dict(B=1, Hq=4, Hkv=1, d=256, N=900, bits_k=2, bits_v=3, wid=118),
    # the bulk encode's strided loads at d = 256: 16-byte segments of fp32
    # inputs and 8-byte segments of fp16 ones, ragged against 8-row items
    "d256_k4v4_f32in_g2": dict(B=1, Hq=4, Hkv=2, d=256, N=333, bits_k=4, bits_v=4,
                               in_dtype="f32", wid=131),
    "d256_k3v3_f16in": dict(B=2, Hq=2, Hkv=1, d=256, N=257, bits_k=3, bits_v=3,
                            in_dtype="f16", wid=132),
    # longer contexts (also the fused appends with long splits, below)
    "d128_k3v4_long": dict(B=1, Hq=8, Hkv=2, N=4000, bits_k=3, bits_v=4, wid=133),
    "d256_k2v3_long": dict(B=1, Hq=4, Hkv=1, d=256, N=3500, bits_k=2, bits_v=3, wid=134),
}


def _run_case(w, scale=0.0, splits=0):
    torch_cuda()
    log(f"case {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} N={w.N} "
        f"K{w.bits_k}/V{w.bits_v} qjl={w.qjl} norm={w.norm_dtype} in={w.in_dtype} "
        f"codebook={w.codebook}")
    cfg, cache = gpu_encode(w)
    ref = oracle_encode(w)
    stats = compare_codes(w, cache, ref)
    qraw, qf = si.queries(w)
    got = gpu_decode(w, cfg, cache, to_device(qraw, w.in_dtype), w.N, scale=scale,
                     splits=splits)
    want = o.attend(qf.astype(np.float64), ref, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k,
                    bits_v=w.bits_v, Hkv=w.Hkv, scale=scale, qjl=w.qjl,
                    qjl_seed=w.qjl_seed, sphere=w.codebook == "sphere")
    err, abs_err = rel_err(got, want)
    log(f"  boundary stats {stats}; max row-relative error {err:.3e} (abs {abs_err:.3e})")
    assert np.isfinite(got).all()
    assert err <= TOL
    return got


@pytest.mark.parametrize("name", sorted(SMALL))
def test_encode_and_decode_match_oracle(name):
    _run_case(si.small_workload(**SMALL[name]))


@pytest.mark.parametrize("name", ["d128_k3v4_gqa4", "d256_k2v2_outlier", "d128_k3v3_g3",
                                  "d128_k3qjl_v4_corr"])
def test_valu_decode_kernel_matches_oracle(name, monkeypatch):
    """TQ_DECODE_VALU=1 sends every format to the VALU decode kernel (no
    matrix cores); it must meet the same bar."""
    monkeypatch.setenv("TQ_DECODE_VALU", "1")
    _run_case(si.small_workload(**SMALL[name]))


def test_explicit_scale():
    _run_case(si.small_workload(B=1, Hq=4, Hkv=2, N=777, wid=120), scale=0.37)


def test_split_count_invariance_and_determinism():
    torch = torch_cuda()
    w = si.small_workload(B=1, Hq=8, Hkv=2, N=3000, bits_k=3, bits_v=4, wid=121)
    cfg, cache = gpu_encode(w)
    qraw, _ = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    base = gpu_decode(w, cfg, cache, q, w.N, splits=1)
    for s in (2, 5, 12, 0):
        other = gpu_decode(w, cfg, cache, q, w.N, splits=s)
        err, _ = rel_err(other, base)
        log(f"splits={s}: rel diff vs 1 split {err:.2e}")
        # the weights enter the value sum as fp16, rounded relative to the
        # running max, and the running max depends on where a split starts
        assert err <= 1e-3
    again = gpu_decode(w, cfg, cache, q, w.N)
    assert np.array_equal(again, gpu_decode(w, cfg, cache, q, w.N))


def test_workspace_reuse_across_calls():
    """One workspace, sized for the largest call, serves calls with different
    split counts and context lengths back to back; each result equals the
    same call on a fresh workspace (the output is poisoned before every
    call, so a merge that did not run shows up)."""
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(B=1, Hq=8, Hkv=2, N=3000, bits_k=3, bits_v=4, wid=128)
    cfg, cache = gpu_encode(w)
    qraw, _ = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    calls = [(3000, 0), (3000, 5), (1700, 2), (3000, 1), (900, 0), (3000, 12), (3000, 5)]
    nbytes = max(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, n, s) for n, s in calls)
    ws = tq.workspace(nbytes)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    for n, s in calls:
        out.fill_(float("nan"))
        tq.tq_attend_decode(cfg, q, cache, n, out, ws, splits=s)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        fresh = gpu_decode(w, cfg, cache, q, n, splits=s)
        log(f"n_ctx={n} splits={s}: reused workspace equals a fresh one")
        assert np.isfinite(got).all()
        assert np.array_equal(got, fresh), (n, s)


APPEND_CASES = ["d128_k3v4_gqa4", "d256_k2v2_outlier", "d128_k4v2_g8", "d128_n1",
                "d128_k4v4_f32norm_f32in_g1", "d128_k3qjl_v4_corr", "d128_k2v3_g2_f16in"]


@pytest.mark.parametrize("name", APPEND_CASES)
def test_append_attend_matches_encode_then_decode(name):
    """tq_append_attend_decode (one launch for 2/4-bit values without QJL,
    encode then decode for the other formats) leaves the same cache bytes
    and the same output as tq_encode_kv of token N-1 followed by
    tq_attend_decode, and the output matches the oracle; split counts 0 and
    3 (the appended token sits in the last split either way)."""
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(**SMALL[name])
    log(f"case {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} N={w.N} K{w.bits_k}/V{w.bits_v} "
        f"qjl={w.qjl}")
    n0 = w.N - 1
    rk, rv, _, _ = kv_host(w, n0, w.N)
    k1, v1 = to_device(rk, w.in_dtype), to_device(rv, w.in_dtype)
    qraw, qf = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    ref = oracle_encode(w)
    want = o.attend(qf.astype(np.float64), ref, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k,
                    bits_v=w.bits_v, Hkv=w.Hkv, qjl=w.qjl, qjl_seed=w.qjl_seed)
    for splits in (0, 3):
        cfg, two = gpu_encode(w, chunks=[(0, n0)] if n0 > 0 else [], capacity=w.N)
        _, one = gpu_encode(w, chunks=[(0, n0)] if n0 > 0 else [], capacity=w.N)
        tq.tq_encode_kv(cfg, k1, v1, n0, two)
        ref_out = gpu_decode(w, cfg, two, q, w.N, splits=splits)
        out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
        ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N, splits))
        tq.tq_append_attend_decode(cfg, k1, v1, q, one, w.N, out, ws, splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        for plane in ("kc", "vc", "kn", "vn", "kq", "kr"):
            a, b = getattr(one, plane), getattr(two, plane)
            if a is None:
                continue
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), plane
        assert np.array_equal(got, ref_out)
        err, _ = rel_err(got, want)
        log(f"  splits={splits}: fused step equals encode + decode; error vs oracle {err:.2e}")
        assert err <= TOL


@pytest.mark.parametrize("name", ["d128_k3v4_long", "d256_k2v3_long"])
def test_fused_appends_with_long_splits(name):
    """With one or two splits of about 2000-4000 tokens, each split holds more
    old tokens than its first tiles ((PF + 1) x 512 tokens), so the fused
    single-token and chunk steps request those tiles before the set-up and
    the encode, as the plain decode does. Both steps against encode + decode
    (cache bytes equal; single token: output bit-identical; chunk: within the
    tolerance) and against the oracle."""
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(**SMALL[name])
    log(f"case {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} N={w.N} K{w.bits_k}/V{w.bits_v}")
    qraw, qf = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    ref = oracle_encode(w)
    want = o.attend(qf.astype(np.float64), ref, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k,
                    bits_v=w.bits_v, Hkv=w.Hkv)
    for n_new in (1, 300):
        n0 = w.N - n_new
        rk, rv, _, _ = kv_host(w, n0, w.N)
        kc, vc = to_device(rk, w.in_dtype), to_device(rv, w.in_dtype)
        for splits in (1, 2):
            cfg, two = gpu_encode(w, chunks=[(0, n0)], capacity=w.N)
            _, one = gpu_encode(w, chunks=[(0, n0)], capacity=w.N)
            tq.tq_encode_kv(cfg, kc, vc, n0, two)
            ref_out = gpu_decode(w, cfg, two, q, w.N, splits=splits)
            out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
            ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N, splits))
            if n_new == 1:
                tq.tq_append_attend_decode(cfg, kc, vc, q, one, w.N, out, ws, splits=splits)
            else:
                tq.tq_append_chunk_attend_decode(cfg, kc, vc, q, one, w.N, out, ws,
                                                 splits=splits)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            for plane in ("kc", "vc", "kn", "vn"):
                assert torch.equal(getattr(one, plane).view(torch.uint8),
                                   getattr(two, plane).view(torch.uint8)), plane
            err, _ = rel_err(got, want)
            diff, _ = rel_err(got, ref_out)
            log(f"  n_new={n_new} splits={splits}: error vs oracle {err:.2e}, "
                f"vs the two calls {diff:.2e}")
            assert err <= TOL
            if n_new == 1:
                assert np.array_equal(got, ref_out)
            else:
                assert diff <= TOL


@pytest.mark.parametrize("splits,scale", [(1, 0.0), (3, 0.0), (1, 0.35), (2, 0.35)])
def test_many_tiles_per_split(splits, scale):
    """Long splits (up to 10 tiles of 512 tokens in one workgroup, every
    rotation of the prefetch buffers, ragged tail) against the oracle; scale
    0.35 widens the score range ~4x so the running max is raised often."""
    _run_case(si.small_workload(B=1, Hq=4, Hkv=1, N=5037, bits_k=3, bits_v=4,
                                structure="correlated", wid=127), scale=scale, splits=splits)


CHUNK_CASES = ["d128_k3v4_gqa4", "d256_k2v2_outlier", "d128_k3v3_g3",
               "d128_k4v4_f32norm_f32in_g1", "d128_k3qjl_v4_corr", "d128_n1"]


@pytest.mark.parametrize("name", CHUNK_CASES)
def test_append_chunk_attend_matches_encode_then_decode(name):
    """tq_append_chunk_attend_decode (one launch on the matrix-core decode
    without QJL: every split encodes and reads a share of the new tokens;
    encode then decode otherwise) leaves the same cache bytes as tq_encode_kv
    of the chunk, and its output matches the oracle and the two-call result
    (bit for bit when it makes the two calls): chunks of 1, 37, 300 and all
    N tokens, split counts 0 and 5."""
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(**SMALL[name])
    fused = not w.qjl
    log(f"case {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} d={w.d} N={w.N} K{w.bits_k}/V{w.bits_v} "
        f"qjl={w.qjl} in={w.in_dtype}")
    qraw, qf = si.queries(w)
    q = to_device(qraw, w.in_dtype)
    ref = oracle_encode(w)
    want = o.attend(qf.astype(np.float64), ref, w.N, d=w.d, seed=w.seed, bits_k=w.bits_k,
                    bits_v=w.bits_v, Hkv=w.Hkv, qjl=w.qjl, qjl_seed=w.qjl_seed)
    for n_new in sorted({1, min(37, w.N), min(300, w.N), w.N}):
        n0 = w.N - n_new
        rk, rv, _, _ = kv_host(w, n0, w.N)
        kc, vc = to_device(rk, w.in_dtype), to_device(rv, w.in_dtype)
        for splits in (0, 5):
            if n0 > 0:
                cfg, two = gpu_encode(w, chunks=[(0, n0)], capacity=w.N)
                _, one = gpu_encode(w, chunks=[(0, n0)], capacity=w.N)
            else:                         # the chunk is the whole context
                cfg = config_of(w)
                two = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
                one = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
            tq.tq_encode_kv(cfg, kc, vc, n0, two)
            ref_out = gpu_decode(w, cfg, two, q, w.N, splits=splits)
            out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
            ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, w.N, splits))
            tq.tq_append_chunk_attend_decode(cfg, kc, vc, q, one, w.N, out, ws, splits=splits)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            for plane in ("kc", "vc", "kn", "vn", "kq", "kr"):
                a, b = getattr(one, plane), getattr(two, plane)
                if a is None:
                    continue
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), plane
            err, _ = rel_err(got, want)
            diff, _ = rel_err(got, ref_out)
            log(f"  n_new={n_new} splits={splits}: error vs oracle {err:.2e}, "
                f"vs the two calls {diff:.2e}")
            assert err <= TOL
            if fused:
                assert diff <= TOL
            else:
                assert np.array_equal(got, ref_out)


def test_append_chunks_equal_bulk_encode():
    """Encoding as several appends writes the same planes as one encode."""
    torch = torch_cuda()
    w = si.small_workload(B=2, Hq=4, Hkv=2, N=700, bits_k=3, bits_v=4, qjl=True, wid=122)
    _, bulk = gpu_encode(w)
    _, parts = gpu_encode(w, chunks=[(0, 1), (1, 300), (300, 301), (301, 700)])
    for name in ("kc", "vc", "kn", "vn", "kq", "kr"):
        assert torch.equal(getattr(bulk, name), getattr(parts, name)), name


def test_decode_prefix_of_larger_cache():
    """n_ctx < capacity attends to the first n_ctx tokens only."""
    w = si.small_workload(B=1, Hq=4, Hkv=2, N=800, wid=123)
    cfg, cache = gpu_encode(w, capacity=1000)
    qraw, qf = si.queries(w)
    n = 517
    got = gpu_decode(w, cfg, cache, to_device(qraw, w.in_dtype), n)
    ref = oracle_encode(w, 0, n)
    want = o.attend(qf.astype(np.float64), ref, n, d=w.d, seed=0, bits_k=3, bits_v=4, Hkv=2)
    assert rel_err(got, want)[0] <= TOL


def test_zero_vectors_encode_and_decode():
    """All-zero key/value rows: norm 0, middle code, zero contribution."""
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(B=1, Hq=2, Hkv=1, N=64, wid=124)
    rk, rv, fk, fv = kv_host(w, 0, w.N)
    rk[:, :, 5] = 0
    rv[:, :, 5] = 0
    rk[:, :, 9] = 0
    fk[:, :, 5] = 0; fv[:, :, 5] = 0; fk[:, :, 9] = 0
    cfg = config_of(w)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, w.N)
    tq.tq_encode_kv(cfg, to_device(rk, "bf16"), to_device(rv, "bf16"), 0, cache)
    torch.cuda.synchronize()
    ref = o.encode_kv(fk, fv, seed=0, bits_k=3, bits_v=4, norm_dtype="f16")
    compare_codes(w, cache, ref)
    assert cache.kn[0, 0, 5].item() == 0 and cache.vn[0, 0, 5].item() == 0
    qraw, qf = si.queries(w)
    got = gpu_decode(w, cfg, cache, to_device(qraw, "bf16"), w.N)
    want = o.attend(qf.astype(np.float64), ref, w.N, d=w.d, seed=0, bits_k=3, bits_v=4, Hkv=1)
    assert rel_err(got, want)[0] <= TOL


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("inverse", [False, True])
def test_rht_matches_oracle(d, dtype, inverse):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    rows = 37
    rng = np.random.default_rng(d + len(dtype))
    x32 = rng.standard_normal((rows, d)).astype(np.float32)
    raw, xf = si._round_input(x32, dtype)
    y = torch.empty((rows, d), dtype=torch.float32, device="cuda")
    tq.tq_rht(to_device(raw, dtype), y, seed=7, inverse=inverse)
    torch.cuda.synchronize()
    fn = o.rht_inverse if inverse else o.rht
    want = fn(xf.astype(np.float64), 7)
    got = y.cpu().numpy().astype(np.float64)
    assert np.abs(got - want).max() <= 1e-6 * np.abs(want).max()


@pytest.mark.parametrize("d", [128, 256])
def test_qjl_sketch_matches_oracle_and_encode(d):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    rows = 50
    rng = np.random.default_rng(d)
    r = (0.2 * rng.standard_normal((rows, d))).astype(np.float32)
    r[3] = 0.0
    bits = torch.empty((rows, d // 32), dtype=torch.int32, device="cuda")
    rn = torch.empty((rows,), dtype=torch.float16, device="cuda")
    tq.tq_qjl_sketch(to_device(r, "f32"), 5, bits, rn)
    torch.cuda.synchronize()
    ref = o.qjl_sketch(r.astype(np.float64), 5)
    got = o.unpack_signs(bits.cpu().numpy().view(np.uint8).reshape(rows, d // 8), d)
    bnd = o.qjl_boundary_mask(ref["w"], ref["rnorm_exact"])
    assert not ((got != ref["bits"]) & ~bnd).any()
    gr = rn.float().cpu().numpy().astype(np.float64)
    amb = o.norm_ambiguous(ref["rnorm_exact"], "f16")
    assert not ((gr != ref["rnorm"]) & ~amb).any()
    assert gr[3] == 0 and not got[3].any()

    # encode with QJL == encode, form the residual, sketch it
    w = si.small_workload(B=1, Hq=2, Hkv=1, d=d, N=40, qjl=True, qjl_seed=5, wid=125)
    cfg, cache = gpu_encode(w)
    _, _, fk, _ = kv_host(w, 0, w.N)
    codes = o.unpack_codes(cache.kc.cpu().numpy(), w.bits_k, d)
    norms = cache.kn.float().cpu().numpy().astype(np.float64)
    res = o.rht(fk, 0) - o.dequant_rot(codes, norms, w.bits_k)
    bits2 = torch.empty((w.N, d // 32), dtype=torch.int32, device="cuda")
    rn2 = torch.empty((w.N,), dtype=torch.float16, device="cuda")
    tq.tq_qjl_sketch(to_device(res.reshape(-1, d).astype(np.float32), "f32"), 5, bits2, rn2)
    torch.cuda.synchronize()
    a = o.unpack_signs(cache.kq.cpu().numpy().reshape(w.N, d // 8), d)
    b = o.unpack_signs(bits2.cpu().numpy().view(np.uint8).reshape(w.N, d // 8), d)
    wv = o.rht(res.reshape(-1, d), 5)
    near = np.abs(wv) < 1e-5 * np.linalg.norm(res.reshape(-1, d), axis=-1, keepdims=True)
    assert not ((a != b) & ~near).any()


def test_dense_bf16_baseline_matches_fp64_attention():
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    w = si.small_workload(B=2, Hq=8, Hkv=2, N=900, wid=126)
    rk, rv, fk, fv = kv_host(w, 0, w.N)
    qraw, qf = si.queries(w)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_dense_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N))
    tq.tq_dense_decode_bf16(to_device(qraw, "bf16"), to_device(rk, "bf16"), to_device(rv, "bf16"),
                            out, ws)
    torch.cuda.synchronize()
    G = w.G
    want = np.zeros((w.B, w.Hq, w.d))
    for b in range(w.B):
        for h in range(w.Hq):
            lg = fk[b, h // G] @ qf[b, h].astype(np.float64) / math.sqrt(w.d)
            p = np.exp(lg - lg.max())
            want[b, h] = (p / p.sum()) @ fv[b, h // G]
    err, _ = rel_err(out.cpu().numpy().astype(np.float64), want)
    assert err <= 1e-4


def test_read_probe_reads_every_word():
    # the XOR of the per-wave words equals the XOR of every 32-bit word of
    # the buffer: each 16-byte chunk was loaded exactly once
    torch = torch_cuda()
    import decode_attention_seeded_amd as tq
    rng = np.random.default_rng(7)
    for nbytes in (16, 4096 + 48, (3 << 20) + 16 * 37):
        host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
        dev = torch.from_numpy(host.view(np.int32)).cuda()
        log(f"read probe: {nbytes} bytes")
        sink = tq.tq_read_probe(dev)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), nbytes
