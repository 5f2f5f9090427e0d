"""C-ABI tests that need no GPU: the library loads, exports what include/tq.h
declares, host helpers agree with the independent oracle, and every argument
check returns its status before any device work. No test here launches a
kernel; paths that would pass validation are only taken with B = 0 or
n_new = 0 (documented no-ops)."""

import ctypes
import json
import math
import os
import re

import numpy as np
import pytest

import decode_attention_seeded_amd as tq
from decode_attention_seeded_amd import binding as bd
import oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "tq.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:const char\*|int64_t|int)\s+(tq_\w+)\s*\(", header, re.M))
    assert declared == set(tq.EXPORTS)
    lib = tq.lib()
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_host_codebook_matches_oracle(bits):
    c, t = tq.tq_codebook(bits)
    oc, ot = o.lloyd_max(bits)
    np.testing.assert_allclose(c, oc, atol=1e-13, rtol=0)
    np.testing.assert_allclose(t, ot, atol=1e-13, rtol=0)
    assert t[len(t) // 2] == 0.0


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_host_sphere_codebook_matches_oracle(bits, d):
    c, t = tq.tq_codebook_ex(bits, "sphere", d)
    oc, ot = o.lloyd_max(bits, d)
    # both sides stop a linearly converging Lloyd iteration at a step of
    # ~1e-13 (different quadratures), which leaves them ~1e-10 apart: far
    # inside the 1e-6 decision-boundary band of every code comparison
    np.testing.assert_allclose(c, oc, atol=1e-9, rtol=0)
    np.testing.assert_allclose(t, ot, atol=1e-9, rtol=0)
    assert t[len(t) // 2] == 0.0
    g, _ = tq.tq_codebook_ex(bits, "gauss", d)
    assert g == tq.tq_codebook(bits)[0]
    with pytest.raises(tq.TqError):
        tq.tq_codebook_ex(bits, "sphere", 64)


LOOKUP_CASES = [(bits, kind, d) for bits in (3, 4)
                for kind, d in (("gauss", 128), ("gauss", 256), ("sphere", 128), ("sphere", 256))]


@pytest.mark.parametrize("bits,kind,d", LOOKUP_CASES)
def test_thresholds_fit_the_encode_lookup(bits, kind, d):
    """The bulk encode finds 3- and 4-bit codes through buckets of width
    1/4 in z = u / n over [-4, 4), the end buckets open: each bucket may hold
    at most one threshold strictly inside it, so consecutive thresholds must
    be more than 1/4 apart, and none may lie in an end bucket."""
    _, t = tq.tq_codebook_ex(bits, kind, d)
    t = np.asarray(t)
    assert len(t) == (1 << bits) - 1 and t[len(t) // 2] == 0.0
    assert (np.diff(t) > 1 / 4).all()
    np.testing.assert_array_equal(t, -t[::-1])      # antisymmetric
    assert np.abs(t).max() < 3.75                    # inside the inner buckets


def _lookup_codes(t, bits, z):
    """The encode's lookup rule, restated: bucket b of 4 z + OFF, clamped
    to [0, 2 OFF), entry 4 t + OFF of the threshold inside it (2^60 if
    none) with its low bits replaced by the count of thresholds at or below
    the bucket's edge."""
    off, scale = 16, 4
    nb = 2 * off
    ent = np.empty(nb, dtype=np.uint64)
    for b in range(nb):
        lo, hi = (b - off) / scale, (b + 1 - off) / scale
        c0 = int((t <= lo).sum())
        inside = t[(t > lo) & (t < hi)]
        assert len(inside) <= 1
        tb = scale * inside[0] + off if len(inside) else 2.0 ** 60
        raw = np.array([tb]).view(np.uint64)[0]
        ent[b] = (raw & ~np.uint64((1 << bits) - 1)) | np.uint64(c0)
    zz = scale * z + off
    idx = np.clip(np.trunc(zz).astype(np.int64), 0, nb - 1)
    e = ent[idx]
    low = (e & np.uint64((1 << bits) - 1)).astype(np.int64) + (zz >= e.view(np.float64))
    return low & ((1 << bits) - 1), low >> bits


@pytest.mark.parametrize("bits,kind,d", LOOKUP_CASES)
def test_encode_lookup_rule_counts_thresholds(bits, kind, d):
    """The lookup gives #{k : z >= t_k} over the whole range |z| <= sqrt(d)
    (beyond the table's [-4, 4) through its clamped end buckets), away from
    the thresholds, and never carries into the bits above the code."""
    _, t = tq.tq_codebook_ex(bits, kind, d)
    t = np.asarray(t)
    rng = np.random.default_rng(bits * 1000 + d)
    z = np.concatenate([rng.uniform(-np.sqrt(d), np.sqrt(d), 20000),
                        rng.standard_normal(20000), t - 1e-7, t + 1e-7, [0.0, -1e-9],
                        np.arange(-20, 21) / 4, [np.sqrt(d), -np.sqrt(d)]])
    got, carry = _lookup_codes(t, bits, z)
    want = (z[:, None] >= t[None, :]).sum(1)
    np.testing.assert_array_equal(got, want)
    assert not carry.any()


@pytest.mark.parametrize("seed,d", [(0, 128), (1, 256), (12345, 128)])
def test_host_signs_match_oracle(seed, d):
    assert tq.tq_signs(seed, d) == list(o.signs(seed, d).astype(int))


def test_bits_split_matches_truth_table():
    with open(os.path.join(ROOT, "tests", "golden", "enable_rule.json")) as f:
        g = json.load(f)
    for bits, scheme, want in g["enabled"]:
        if bits is None:
            continue
        got = tq.tq_bits_split(bits, scheme == "turboquant")
        assert (got is not None) == want, (bits, scheme)
        if want:
            assert got == o.bits_split(bits, scheme)
    assert tq.tq_bits_split(3.5) == (3, 4)
    with pytest.raises(tq.TqError) as e:
        tq.tq_bits_split(5.5)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    with pytest.raises(tq.TqError):
        tq.tq_bits_split(float("nan"))


@pytest.mark.parametrize("bk,bv,nd,qjl,d", [(3, 4, "f16", False, 128), (4, 4, "f32", False, 128),
                                            (2, 2, "f16", False, 256), (3, 4, "f16", True, 128)])
def test_cache_bytes_match_format(bk, bv, nd, qjl, d):
    cfg = tq.Config(d=d, bits_k=bk, bits_v=bv, norm_dtype=nd, qjl=qjl)
    total, planes = tq.tq_cache_bytes(cfg, 2, 3, 100)
    nb = 2 if nd == "f16" else 4
    assert total == 600 * o.tq_bytes_per_token(d, bk, bv, nb, qjl)
    assert planes[0] == 600 * d * bk // 8 and planes[1] == 600 * d * bv // 8


def test_split_plan_and_workspace(monkeypatch):
    cfg = tq.Config(d=128, bits_k=3, bits_v=4)
    s = tq.tq_num_splits(cfg, 1, 32, 8, 524288)
    assert s >= 8
    assert tq.tq_num_splits(cfg, 1, 32, 8, 1) == 1
    # clamped to tiles: workgroup rounds are 64 tokens per wave; the
    # matrix-core kernel (d 128 / 256, with or without QJL) runs 8 waves; the
    # VALU kernel (TQ_DECODE_VALU=1, or other head dims) uses 256-token tiles
    # at d 128
    assert tq.tq_num_splits(cfg, 1, 32, 8, 300, splits=7) == 1
    assert tq.tq_num_splits(cfg, 1, 32, 8, 2100, splits=7) == 5
    cfgq = tq.Config(d=128, bits_k=3, bits_v=4, qjl=True)
    assert tq.tq_num_splits(cfgq, 1, 32, 8, 2100, splits=7) == 5
    cfg256 = tq.Config(d=256, bits_k=2, bits_v=2)
    assert tq.tq_num_splits(cfg256, 8, 16, 4, 1100, splits=7) == 3
    cfg3 = tq.Config(d=128, bits_k=3, bits_v=3)
    assert tq.tq_num_splits(cfg3, 1, 32, 8, 300, splits=7) == 1
    monkeypatch.setenv("TQ_DECODE_VALU", "1")
    assert tq.tq_num_splits(cfg3, 1, 32, 8, 300, splits=7) == 2
    assert tq.tq_num_splits(cfg, 1, 32, 8, 300, splits=7) == 2
    monkeypatch.delenv("TQ_DECODE_VALU")
    # default: one round of ~256 workgroups for the wave-private kernels
    assert s == 32
    ws = tq.tq_workspace_bytes(cfg, 1, 32, 8, 524288)
    assert ws >= 32 * 128 * 4 + 32 * s * (128 + 2) * 4
    with pytest.raises(tq.TqError) as e:
        tq.tq_num_splits(cfg, 1, 30, 8, 100)
    assert e.value.status == tq.TQ_ERR_ARG


def test_strerror_names_every_status():
    for s in range(0, -8, -1):
        assert tq.tq_strerror(s).startswith("TQ_")
    assert tq.tq_strerror(-99) == "unknown tq_status"


# ---------------------------------------------------------------- validation
# Fake device addresses: aligned (0x1000...) and misaligned (+4). They are
# never dereferenced: every call below fails validation or is a no-op.

A = 0x10000
MIS = 0x10004


def _cfg(**kw):
    base = dict(d=128, bits_k=3, bits_v=4, norm_dtype=tq.TQ_F16, qjl=0, seed=0, qjl_seed=1)
    base.update(kw)
    return bd.tq_config(**base)


def _cache(B=1, Hkv=2, cap=64, **kw):
    c = bd.tq_cache(A, A, A, A, A, A, B, Hkv, cap)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _enc(cfg=None, k=A, v=A, dt=tq.TQ_BF16, off=0, n=4, cache=None):
    lib = tq.lib()
    cfg = _cfg() if cfg is None else cfg
    cache = _cache() if cache is None else cache
    return lib.tq_encode_kv(ctypes.byref(cfg) if cfg != "null" else None, k, v, dt, off, n,
                            ctypes.byref(cache) if cache != "null" else None, None)


def test_codebook_kind_validation():
    assert _enc(cfg=_cfg(codebook=2)) == tq.TQ_ERR_UNSUPPORTED
    assert _enc(cfg=_cfg(codebook=1), n=0) == tq.TQ_OK


def test_encode_validation():
    assert _enc(cfg="null") == tq.TQ_ERR_ARG
    assert _enc(cfg=_cfg(d=64)) == tq.TQ_ERR_UNSUPPORTED
    assert _enc(cfg=_cfg(bits_k=5)) == tq.TQ_ERR_UNSUPPORTED
    assert _enc(cfg=_cfg(bits_v=1)) == tq.TQ_ERR_UNSUPPORTED
    assert _enc(cfg=_cfg(norm_dtype=tq.TQ_BF16)) == tq.TQ_ERR_UNSUPPORTED
    assert _enc(cfg=_cfg(qjl=2)) == tq.TQ_ERR_ARG
    assert _enc(cache="null") == tq.TQ_ERR_ARG
    assert _enc(cache=_cache(kc=None)) == tq.TQ_ERR_ARG
    assert _enc(cache=_cache(vn=MIS)) == tq.TQ_ERR_ALIGN
    assert _enc(cfg=_cfg(qjl=1), cache=_cache(kq=None)) == tq.TQ_ERR_ARG
    assert _enc(cfg=_cfg(qjl=1), cache=_cache(kr=MIS)) == tq.TQ_ERR_ALIGN
    assert _enc(dt=7) == tq.TQ_ERR_UNSUPPORTED
    assert _enc(off=-1) == tq.TQ_ERR_ARG
    assert _enc(n=-1) == tq.TQ_ERR_ARG
    assert _enc(off=60, n=5) == tq.TQ_ERR_CAPACITY
    assert _enc(k=None) == tq.TQ_ERR_ARG
    assert _enc(v=MIS) == tq.TQ_ERR_ALIGN
    assert _enc(cache=_cache(Hkv=0)) == tq.TQ_ERR_ARG
    assert _enc(n=0) == tq.TQ_OK                       # empty append: no-op
    assert _enc(cache=_cache(B=0)) == tq.TQ_OK         # empty batch: no-op


def _dec(cfg=None, q=A, qdt=tq.TQ_BF16, B=1, Hq=4, cache=None, n_ctx=10, scale=0.0,
         splits=0, out=A, ws=A, ws_bytes=1 << 30):
    lib = tq.lib()
    cfg = _cfg() if cfg is None else cfg
    cache = _cache() if cache is None else cache
    return lib.tq_attend_decode(ctypes.byref(cfg), q, qdt, B, Hq, ctypes.byref(cache), n_ctx,
                                scale, splits, out, ws, ws_bytes, None)


def test_decode_validation():
    assert _dec(cfg=_cfg(d=96)) == tq.TQ_ERR_UNSUPPORTED
    assert _dec(qdt=5) == tq.TQ_ERR_UNSUPPORTED
    assert _dec(B=2) == tq.TQ_ERR_ARG                  # B must match the cache
    assert _dec(Hq=3) == tq.TQ_ERR_ARG                 # Hq % Hkv
    assert _dec(splits=-1) == tq.TQ_ERR_ARG
    assert _dec(scale=float("nan")) == tq.TQ_ERR_ARG
    assert _dec(n_ctx=0) == tq.TQ_ERR_ARG
    assert _dec(n_ctx=65) == tq.TQ_ERR_CAPACITY
    assert _dec(q=None) == tq.TQ_ERR_ARG
    assert _dec(out=MIS) == tq.TQ_ERR_ALIGN
    assert _dec(ws=MIS) == tq.TQ_ERR_ALIGN
    assert _dec(ws_bytes=64) == tq.TQ_ERR_WORKSPACE
    assert _dec(cache=_cache(kn=MIS)) == tq.TQ_ERR_ALIGN
    assert _dec(B=0, cache=_cache(B=0)) == tq.TQ_OK    # empty batch: no-op


def _app(cfg=None, k=A, v=A, dt=tq.TQ_BF16, q=A, qdt=tq.TQ_BF16, B=1, Hq=4, cache=None,
         n_ctx=10, scale=0.0, splits=0, out=A, ws=A, ws_bytes=1 << 30):
    lib = tq.lib()
    cfg = _cfg() if cfg is None else cfg
    cache = _cache() if cache is None else cache
    return lib.tq_append_attend_decode(ctypes.byref(cfg) if cfg != "null" else None, k, v, dt,
                                       q, qdt, B, Hq, ctypes.byref(cache), n_ctx, scale, splits,
                                       out, ws, ws_bytes, None)


def test_append_attend_validation():
    """Both halves of the fused step are checked before anything is queued:
    the encode side (rows, dtype, alignment) and the decode side."""
    assert _app(cfg="null") == tq.TQ_ERR_ARG
    assert _app(cfg=_cfg(bits_v=1)) == tq.TQ_ERR_UNSUPPORTED
    assert _app(cache=_cache(vc=None)) == tq.TQ_ERR_ARG
    assert _app(dt=7) == tq.TQ_ERR_UNSUPPORTED
    assert _app(k=None) == tq.TQ_ERR_ARG
    assert _app(v=MIS) == tq.TQ_ERR_ALIGN
    assert _app(n_ctx=0) == tq.TQ_ERR_ARG
    assert _app(n_ctx=65) == tq.TQ_ERR_CAPACITY
    assert _app(B=2) == tq.TQ_ERR_ARG
    assert _app(qdt=5) == tq.TQ_ERR_UNSUPPORTED
    assert _app(Hq=3) == tq.TQ_ERR_ARG
    assert _app(q=None) == tq.TQ_ERR_ARG
    assert _app(out=MIS) == tq.TQ_ERR_ALIGN
    assert _app(ws_bytes=64) == tq.TQ_ERR_WORKSPACE
    assert _app(cfg=_cfg(qjl=1), cache=_cache(kq=None)) == tq.TQ_ERR_ARG
    assert _app(B=0, cache=_cache(B=0)) == tq.TQ_OK    # empty batch: no-op


def _chunk(cfg=None, k=A, v=A, dt=tq.TQ_BF16, n_new=4, q=A, qdt=tq.TQ_BF16, B=1, Hq=4,
           cache=None, n_ctx=10, scale=0.0, splits=0, out=A, ws=A, ws_bytes=1 << 30):
    lib = tq.lib()
    cfg = _cfg() if cfg is None else cfg
    cache = _cache() if cache is None else cache
    return lib.tq_append_chunk_attend_decode(ctypes.byref(cfg) if cfg != "null" else None, k, v,
                                             dt, n_new, q, qdt, B, Hq, ctypes.byref(cache),
                                             n_ctx, scale, splits, out, ws, ws_bytes, None)


def test_append_chunk_attend_validation():
    """The chunked step checks the chunk (1 <= n_new <= n_ctx, rows, dtype,
    alignment) and the decode side before anything is queued."""
    assert _chunk(cfg="null") == tq.TQ_ERR_ARG
    assert _chunk(cfg=_cfg(bits_k=5)) == tq.TQ_ERR_UNSUPPORTED
    assert _chunk(cache=_cache(kc=None)) == tq.TQ_ERR_ARG
    assert _chunk(dt=7) == tq.TQ_ERR_UNSUPPORTED
    assert _chunk(n_new=0) == tq.TQ_ERR_ARG
    assert _chunk(n_new=11) == tq.TQ_ERR_ARG              # more new tokens than the context
    assert _chunk(n_ctx=0) == tq.TQ_ERR_ARG
    assert _chunk(n_ctx=65, n_new=4) == tq.TQ_ERR_CAPACITY
    assert _chunk(k=None) == tq.TQ_ERR_ARG
    assert _chunk(v=MIS) == tq.TQ_ERR_ALIGN
    assert _chunk(B=2) == tq.TQ_ERR_ARG
    assert _chunk(qdt=5) == tq.TQ_ERR_UNSUPPORTED
    assert _chunk(Hq=3) == tq.TQ_ERR_ARG
    assert _chunk(q=None) == tq.TQ_ERR_ARG
    assert _chunk(out=MIS) == tq.TQ_ERR_ALIGN
    assert _chunk(ws_bytes=64) == tq.TQ_ERR_WORKSPACE
    assert _chunk(B=0, cache=_cache(B=0)) == tq.TQ_OK    # empty batch: no-op


def test_rht_qjl_dense_validation():
    lib = tq.lib()
    assert lib.tq_rht(A, tq.TQ_F32, A, -1, 128, 0, 0, None) == tq.TQ_ERR_ARG
    assert lib.tq_rht(A, tq.TQ_F32, A, 4, 64, 0, 0, None) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_rht(A, 9, A, 4, 128, 0, 0, None) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_rht(A, tq.TQ_F32, A, 4, 128, 0, 3, None) == tq.TQ_ERR_ARG
    assert lib.tq_rht(None, tq.TQ_F32, A, 4, 128, 0, 0, None) == tq.TQ_ERR_ARG
    assert lib.tq_rht(MIS, tq.TQ_F32, A, 4, 128, 0, 0, None) == tq.TQ_ERR_ALIGN
    assert lib.tq_rht(A, tq.TQ_F32, A, 0, 128, 0, 0, None) == tq.TQ_OK
    assert lib.tq_qjl_sketch(A, 4, 100, 1, A, A, None) == tq.TQ_ERR_UNSUPPORTED
    assert lib.tq_qjl_sketch(A, -2, 128, 1, A, A, None) == tq.TQ_ERR_ARG
    assert lib.tq_qjl_sketch(A, 4, 128, 1, None, A, None) == tq.TQ_ERR_ARG
    assert lib.tq_qjl_sketch(A, 4, 128, 1, A, MIS, None) == tq.TQ_ERR_ALIGN
    assert lib.tq_qjl_sketch(A, 0, 128, 1, A, A, None) == tq.TQ_OK
    bad_d = (A, A, A, 1, 4, 2, 100, 10, 0.0, 0, A, A, 1 << 30, None)
    assert lib.tq_dense_decode_bf16(*bad_d) == tq.TQ_ERR_UNSUPPORTED
    bad_g = (A, A, A, 1, 5, 2, 128, 10, 0.0, 0, A, A, 1 << 30, None)
    assert lib.tq_dense_decode_bf16(*bad_g) == tq.TQ_ERR_ARG
    small = (A, A, A, 1, 4, 2, 128, 10, 0.0, 0, A, A, 8, None)
    assert lib.tq_dense_decode_bf16(*small) == tq.TQ_ERR_WORKSPACE
    mis = (A, MIS, A, 1, 4, 2, 128, 10, 0.0, 0, A, A, 1 << 30, None)
    assert lib.tq_dense_decode_bf16(*mis) == tq.TQ_ERR_ALIGN


def test_read_probe_validation():
    lib = tq.lib()
    assert lib.tq_read_probe(A, -16, A, None) == tq.TQ_ERR_ARG
    assert lib.tq_read_probe(A, 24, A, None) == tq.TQ_ERR_ARG
    assert lib.tq_read_probe(None, 32, A, None) == tq.TQ_ERR_ARG
    assert lib.tq_read_probe(A, 32, None, None) == tq.TQ_ERR_ARG
    assert lib.tq_read_probe(MIS, 32, A, None) == tq.TQ_ERR_ALIGN
    assert lib.tq_read_probe(A, 0, A, None) == tq.TQ_OK
    # one word per wave: 4 per 256-thread block, at most 16384 blocks
    assert lib.tq_read_probe_sink_words(16) == 4
    assert lib.tq_read_probe_sink_words(16 * 256 * 3) == 12
    assert lib.tq_read_probe_sink_words(1 << 40) == 4 * 16384


def test_prefill_validation():
    lib = tq.lib()

    def call(cfg=None, q=A, qdt=tq.TQ_BF16, B=1, Hq=4, n_q=8, cache=None, n_ctx=16, out=A):
        cfg = _cfg() if cfg is None else cfg
        cache = _cache() if cache is None else cache
        return lib.tq_attend_prefill(ctypes.byref(cfg), q, qdt, B, Hq, n_q, ctypes.byref(cache),
                                     n_ctx, 0.0, out, None)

    assert call(cfg=_cfg(qjl=1), cache=_cache(kr=MIS)) == tq.TQ_ERR_ALIGN
    assert call(cfg=_cfg(qjl=1), cache=_cache(kq=None)) == tq.TQ_ERR_ARG
    assert call(cfg=_cfg(d=64)) == tq.TQ_ERR_UNSUPPORTED
    assert call(qdt=7) == tq.TQ_ERR_UNSUPPORTED
    assert call(n_q=0) == tq.TQ_ERR_ARG
    assert call(n_q=17) == tq.TQ_ERR_ARG                  # more queries than positions
    assert call(Hq=3) == tq.TQ_ERR_ARG                    # not a multiple of Hkv
    assert call(B=2) == tq.TQ_ERR_ARG                     # cache holds B = 1
    assert call(n_ctx=65) == tq.TQ_ERR_CAPACITY
    big = 1 << 31                                        # positions past 32 bits
    assert call(n_ctx=big, cache=_cache(cap=big)) == tq.TQ_ERR_UNSUPPORTED
    assert call(q=None) == tq.TQ_ERR_ARG
    assert call(q=MIS) == tq.TQ_ERR_ALIGN
    assert call(out=MIS) == tq.TQ_ERR_ALIGN
    assert call(B=0, cache=_cache(B=0)) == tq.TQ_OK


def test_affine_sizes_and_validation():
    cfg = tq.AffineConfig(d=128, bits_k=4, bits_v=4, group=64, seed=3)
    total, planes = tq.tq_affine_cache_bytes(cfg, 2, 8, 100)
    assert planes == [2 * 8 * 100 * 64, 2 * 8 * 100 * 64] + [2 * 8 * 100 * 2 * 2] * 4
    assert total == 2 * 8 * 100 * o.affine_cache_bytes_per_token(128, 4, 4)
    lib = tq.lib()
    for bad in (dict(group=32), dict(bits_k=5), dict(bits_v=1), dict(d=64)):
        c = tq.AffineConfig(**{**dict(d=128, bits_k=4, bits_v=4, group=64), **bad})
        assert lib.tq_affine_cache_bytes(ctypes.byref(c.c()), 1, 1, 1, None) == tq.TQ_ERR_UNSUPPORTED
    c = ctypes.byref(cfg.c())
    assert lib.tq_affine_num_splits(c, 1, 32, 8, 524288, 0) >= 1
    assert lib.tq_affine_num_splits(c, 1, 30, 8, 1000, 0) == tq.TQ_ERR_ARG      # Hq % Hkv
    assert lib.tq_affine_workspace_bytes(c, 1, 8, 8, 0, 0) == tq.TQ_ERR_ARG     # n_ctx 0
    # splits never exceed one per workgroup round (512 tokens on the
    # matrix-core kernel, which K4/V4 at d 128 runs; 256 on the VALU kernel);
    # tokens per split are whole rounds
    assert lib.tq_affine_num_splits(c, 1, 8, 8, 300, 1000) == 1
    assert lib.tq_affine_num_splits(c, 1, 8, 8, 1100, 1000) == 3
    c3 = ctypes.byref(tq.AffineConfig(d=128, bits_k=4, bits_v=3, group=64, seed=3).c())
    assert lib.tq_affine_num_splits(c3, 1, 8, 8, 300, 1000) == 2
    cache = tq.tq_affine_cache(16, 16, 16, 16, 16, 16, 1, 1, 10)
    q = out = ws = ctypes.c_void_p(16)
    st = lib.tq_affine_attend_decode(c, q, 0, 1, 1, ctypes.byref(cache), 11, 0.0, 0, out, ws,
                                     1 << 20, None)
    assert st == tq.TQ_ERR_CAPACITY
    st = lib.tq_affine_attend_decode(c, q, 0, 1, 1, ctypes.byref(cache), 10, 0.0, 0, out, ws,
                                     16, None)
    assert st == tq.TQ_ERR_WORKSPACE
    st = lib.tq_affine_encode_kv(c, q, q, 0, 5, 6, ctypes.byref(cache), None)
    assert st == tq.TQ_ERR_CAPACITY
    bad_align = tq.tq_affine_cache(16, 17, 16, 16, 16, 16, 1, 1, 10)
    st = lib.tq_affine_encode_kv(c, q, q, 0, 0, 1, ctypes.byref(bad_align), None)
    assert st == tq.TQ_ERR_ALIGN
    assert lib.tq_affine_encode_kv(c, q, q, 0, 0, 0, ctypes.byref(cache), None) == tq.TQ_OK
