"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, run the oracle on the same inputs, compare.

The oracle only ever sees the seeded inputs (never a GPU result); GPU outputs
are unpacked with the oracle's unpacker purely to compare them."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest

import oracle as o
import seeded_inputs as si


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(raw: np.ndarray, in_dtype: str):
    torch = torch_cuda()
    if in_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()
    if in_dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(raw)).cuda()
    return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).cuda()


def kv_host(w: si.Workload, t0: int, t1: int):
    """(raw K, raw V, f64 K, f64 V) of tokens [t0, t1) for all (b, h)."""
    rk, rv, fk, fv = [], [], [], []
    for b in range(w.B):
        for h in range(w.Hkv):
            a, fa = si.kv_rows(w, si.T_K, b, h, t0, t1)
            c, fc = si.kv_rows(w, si.T_V, b, h, t0, t1)
            rk.append(a); rv.append(c); fk.append(fa); fv.append(fc)
    shp = (w.B, w.Hkv, t1 - t0, w.d)
    return (np.stack(rk).reshape(shp), np.stack(rv).reshape(shp),
            np.stack(fk).reshape(shp).astype(np.float64),
            np.stack(fv).reshape(shp).astype(np.float64))


def config_of(w: si.Workload):
    import decode_attention_seeded_amd as tq
    return tq.Config(d=w.d, bits_k=w.bits_k, bits_v=w.bits_v, norm_dtype=w.norm_dtype,
                     qjl=w.qjl, seed=w.seed, qjl_seed=w.qjl_seed, codebook=w.codebook)


def gpu_encode(w: si.Workload, chunks=None, capacity=None):
    """Encode the whole context on the GPU (optionally as several appends)."""
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    cfg = config_of(w)
    cache = tq.PackedCache(cfg, w.B, w.Hkv, capacity or w.N)
    bounds = chunks or [(0, w.N)]
    for t0, t1 in bounds:
        rk, rv, _, _ = kv_host(w, t0, t1)
        k, v = to_device(rk, w.in_dtype), to_device(rv, w.in_dtype)
        tq.tq_encode_kv(cfg, k, v, t0, cache)
    torch.cuda.synchronize()
    return cfg, cache


def oracle_encode(w: si.Workload, t0=0, t1=None):
    t1 = w.N if t1 is None else t1
    _, _, fk, fv = kv_host(w, t0, t1)
    return o.encode_kv(fk, fv, seed=w.seed, bits_k=w.bits_k, bits_v=w.bits_v,
                       norm_dtype=w.norm_dtype, qjl=w.qjl, qjl_seed=w.qjl_seed,
                       sphere=w.codebook == "sphere")


def compare_codes(w, cache, ref, t0=0, t1=None):
    """Bit-exact code/norm/sketch comparison; returns counts of tolerated
    boundary cases. Asserts no mismatch outside them."""
    t1 = w.N if t1 is None else t1
    sl = (slice(None), slice(None), slice(t0, t1))
    stats = {}
    for side, bits in (("k", w.bits_k), ("v", w.bits_v)):
        enc = ref[f"{side}_enc"]
        got = o.unpack_codes(getattr(cache, f"{side}c")[sl].cpu().numpy(), bits, w.d)
        _, thr = o.lloyd_max(bits, w.d if w.codebook == "sphere" else None)
        bnd = o.boundary_mask(enc["z"], thr)
        bad = (got != enc["codes"]) & ~bnd
        assert not bad.any(), f"{side} codes differ at {np.argwhere(bad)[:5]}"
        stats[f"{side}_boundary"] = int(bnd.sum())
        stats[f"{side}_flips_at_boundary"] = int(((got != enc["codes"]) & bnd).sum())
        gn = getattr(cache, f"{side}n")[sl].float().cpu().numpy().astype(np.float64)
        amb = o.norm_ambiguous(enc["norm_exact"], w.norm_dtype)
        badn = (gn != enc["norm"]) & ~amb
        assert not badn.any(), f"{side} norms differ at {np.argwhere(badn)[:5]}"
        stats[f"{side}_norm_ambiguous"] = int(amb.sum())
    if w.qjl:
        sk = ref["k_qjl"]
        got = o.unpack_signs(cache.kq[sl].cpu().numpy(), w.d)
        bnd = o.qjl_boundary_mask(sk["w"], sk["rnorm_exact"])
        # a row whose codes flipped at a boundary has a different residual
        _, thr = o.lloyd_max(w.bits_k, w.d if w.codebook == "sphere" else None)
        row_flip = (o.boundary_mask(ref["k_enc"]["z"], thr)).any(-1, keepdims=True)
        bad = (got != sk["bits"]) & ~bnd & ~row_flip
        assert not bad.any(), f"qjl bits differ at {np.argwhere(bad)[:5]}"
        gr = cache.kr[sl].float().cpu().numpy().astype(np.float64)
        amb = o.norm_ambiguous(sk["rnorm_exact"], "f16") | row_flip[..., 0]
        badr = (gr != sk["rnorm"]) & ~amb
        assert not badr.any(), f"qjl residual norms differ at {np.argwhere(badr)[:5]}"
        stats["qjl_boundary"] = int(bnd.sum())
    return stats


def gpu_decode(w, cfg, cache, q_dev, n_ctx, scale=0.0, splits=0):
    import decode_attention_seeded_amd as tq
    torch = torch_cuda()
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
    ws = tq.workspace(tq.tq_workspace_bytes(cfg, w.B, w.Hq, w.Hkv, n_ctx, splits))
    tq.tq_attend_decode(cfg, q_dev, cache, n_ctx, out, ws, scale=scale, splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    """max over (b, h) of ||got - ref||_inf / ||ref||_inf, and the max
    elementwise absolute error."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / den).max()), float(np.abs(got - ref).max())


TOL = 2e-3
