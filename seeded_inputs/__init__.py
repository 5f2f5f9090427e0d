"""Seeded synthetic inputs for the TurboQuant decode workloads.

This module is shared by the CPU oracle's tests and the HIP path's tests and
benchmark. It holds no arithmetic of the method itself: it only draws the
query, key and value tensors (and rounds them to the input dtype).

Recipe
------
* Every tensor is drawn in blocks of BLOCK tokens. Each (workload, tensor,
  batch, kv-head, block) gets its own NumPy Philox stream keyed by
  SeedSequence([data_seed, workload_id, tensor_id, b, h, block]). Any token
  range can therefore be regenerated on its own, by either side, without
  materialising the whole tensor.
* Values are float32 N(0,1) (NumPy's standard_normal), then rounded
  to-nearest-even to bfloat16 where the workload's inputs are bf16.
* Outlier workload: per (b, kv-head) four distinct channels are drawn from a
  stream of their own and those key channels are multiplied by 20 before the
  rounding; values stay N(0,1).
* Correlated-query workload: per query head a token j is drawn uniformly from
  [0, N) within its KV head (floor(h / G)), and q = 0.8 * k_j + 0.6 * eps with
  eps ~ N(0, I), computed in float32 from the bf16 key and rounded to bf16.

bf16 tensors are carried as uint16 bit patterns (NumPy has no bfloat16).
"""

from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

BLOCK = 65536
DATA_SEED = 0

T_Q, T_K, T_V, T_OUTLIER, T_QJ, T_EPS = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, formats and input structure."""
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int
    bits_k: int
    bits_v: int
    norm_dtype: str          # "f16" | "f32"
    qjl: bool
    in_dtype: str            # "f32" | "bf16" | "f16"
    structure: str           # "iid" | "outlier" | "correlated"
    append: int = 0          # tokens appended at the end of the context
    seed: int = 0            # RHT sign seed
    qjl_seed: int = 1
    codebook: str = "gauss"  # "gauss" | "sphere"

    @property
    def G(self):
        return self.Hq // self.Hkv


WORKLOADS = {
    1: Workload(1, "single-head d128 ctx4096 K4V4 fp32-norm", 1, 1, 1, 128,
                4096, 4, 4, "f32", False, "f32", "iid"),
    2: Workload(2, "gqa32/8 d128 ctx32768 K3V4", 1, 32, 8, 128, 32768, 3, 4,
                "f16", False, "bf16", "iid"),
    3: Workload(3, "outlier-keys b8 16/4 d256 ctx131072 K2V2", 8, 16, 4, 256,
                131072, 2, 2, "f16", False, "bf16", "outlier"),
    4: Workload(4, "long-context 32/8 d128 ctx524288 K3V4 append4096", 1, 32,
                8, 128, 524288, 3, 4, "f16", False, "bf16", "iid",
                append=4096),
    5: Workload(5, "qjl b4 32/8 d128 ctx131072 K3+QJL V4", 4, 32, 8, 128,
                131072, 3, 4, "f16", True, "bf16", "correlated"),
}


def _gen(*keys):
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(
        [int(k) for k in keys])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to nearest-even bfloat16; returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    nan = np.isnan(x)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(w: Workload, b: int, h: int, data_seed=DATA_SEED):
    return np.sort(_gen(data_seed, w.wid, T_OUTLIER, b, h).choice(w.d, 4, replace=False))


def _block_f32(w: Workload, tensor: int, b: int, h: int, blk: int, data_seed):
    n = min(BLOCK, w.N - blk * BLOCK)
    x = _gen(data_seed, w.wid, tensor, b, h, blk).standard_normal(
        (n, w.d), dtype=np.float32)
    if tensor == T_K and w.structure == "outlier":
        x[:, outlier_channels(w, b, h, data_seed)] *= np.float32(20.0)
    return x


def kv_rows(w: Workload, tensor: int, b: int, h: int, t0: int, t1: int,
            data_seed=DATA_SEED):
    """Rows [t0, t1) of K (tensor=T_K) or V (T_V) for (b, kv-head h).

    Returns (raw, f32): raw is float32 for fp32 inputs or uint16 bf16 bits;
    f32 holds the exact input values as float32.
    """
    parts = []
    for blk in range(t0 // BLOCK, (max(t1, t0 + 1) - 1) // BLOCK + 1):
        x = _block_f32(w, tensor, b, h, blk, data_seed)
        lo = max(t0 - blk * BLOCK, 0)
        hi = min(t1 - blk * BLOCK, x.shape[0])
        parts.append(x[lo:hi])
    x = np.concatenate(parts) if parts else np.zeros((0, w.d), np.float32)
    return _round_input(x, w.in_dtype)


def _round_input(x: np.ndarray, in_dtype: str):
    if in_dtype == "bf16":
        raw = f32_to_bf16_bits(x)
        return raw, bf16_bits_to_f32(raw)
    if in_dtype == "f16":
        raw = x.astype(np.float16)
        return raw, raw.astype(np.float32)
    return x, x


def queries(w: Workload, data_seed=DATA_SEED):
    """q [B][Hq][d] as (raw, f32); see the module docstring for the recipe."""
    if w.structure != "correlated":
        x = _gen(data_seed, w.wid, T_Q, 0, 0, 0).standard_normal(
            (w.B, w.Hq, w.d), dtype=np.float32)
    else:
        x = np.empty((w.B, w.Hq, w.d), np.float32)
        js = correlated_tokens(w, data_seed)
        eps = _gen(data_seed, w.wid, T_EPS, 0, 0, 0).standard_normal(
            (w.B, w.Hq, w.d), dtype=np.float32)
        for b in range(w.B):
            for hq in range(w.Hq):
                j = int(js[b, hq])
                _, kj = kv_rows(w, T_K, b, hq // w.G, j, j + 1, data_seed)
                x[b, hq] = np.float32(0.8) * kj[0] + np.float32(0.6) * eps[b, hq]
    return _round_input(x, w.in_dtype)


def chunk_queries(w: Workload, n_q: int, data_seed=DATA_SEED):
    """Queries of a prefill chunk, q [B][Hq][n_q][d] iid N(0,1) in the
    workload's input dtype, as (raw, f32)."""
    x = _gen(data_seed, w.wid, T_Q, 1, n_q, 0).standard_normal(
        (w.B, w.Hq, n_q, w.d), dtype=np.float32)
    return _round_input(x, w.in_dtype)


def correlated_tokens(w: Workload, data_seed=DATA_SEED):
    """Token index j per (b, query head) for the correlated-query workload."""
    return _gen(data_seed, w.wid, T_QJ, 0, 0, 0).integers(0, w.N, size=(w.B, w.Hq))


def kv_full(w: Workload, tensor: int, data_seed=DATA_SEED, workers=None):
    """Whole K or V tensor [B][Hkv][N][d] as raw (uint16 bf16 bits or f32).

    Blocks are generated on a thread pool (NumPy releases the GIL in its
    generators), so a 1 GiB tensor takes seconds.
    """
    dt = {"bf16": np.uint16, "f16": np.float16}.get(w.in_dtype, np.float32)
    out = np.empty((w.B, w.Hkv, w.N, w.d), dt)
    jobs = [(b, h, blk) for b in range(w.B) for h in range(w.Hkv)
            for blk in range((w.N + BLOCK - 1) // BLOCK)]

    def run(job):
        b, h, blk = job
        t0 = blk * BLOCK
        t1 = min(w.N, t0 + BLOCK)
        raw, _ = kv_rows(w, tensor, b, h, t0, t1, data_seed)
        out[b, h, t0:t1] = raw

    n = workers or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(n) as ex:
        list(ex.map(run, jobs))
    return out


def small_workload(B=1, Hq=4, Hkv=2, d=128, N=300, bits_k=3, bits_v=4,
                   norm_dtype="f16", qjl=False, in_dtype="bf16",
                   structure="iid", wid=100, seed=0, qjl_seed=1, codebook="gauss"):
    """A small workload for parity tests (several tiles and a ragged tail)."""
    return Workload(wid, f"small-{wid}", B, Hq, Hkv, d, N, bits_k, bits_v,
                    norm_dtype, qjl, in_dtype, structure, seed=seed,
                    qjl_seed=qjl_seed, codebook=codebook)
