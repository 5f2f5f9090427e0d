"""Group-affine KV cache with rotated keys: CPU oracle.

TEST INFRASTRUCTURE ONLY (same rule as the rest of this package: the product
path never imports it).

Follows the "mlx-turboquant" README: "Quantize the KV cache" (make_prompt_cache
with kv_bits and kv_group_size = 64), "How it plugs in" (the KV cache is a
subclass of mlx-lm's quantized, i.e. group-affine, cache; it rotates the keys,
and the patched attention rotates the query) and the "Memory footprint" table
(affine 4-bit and TurboQuant 4-bit at the same bytes per token: d*bits/8 code
bytes plus an fp16 scale and an fp16 bias per group of 64).

READINGS (the README fixes neither formula):
* affine code of a group x_1..x_G with b bits: bias = min x, scale =
  (max x - min x) / (2^b - 1), both stored as fp16 (round to nearest even);
  the code is the nearest level of the stored grid, round((x - bias16) /
  scale16) clamped to [0, 2^b - 1] (ties to even); scale16 == 0 gives code 0.
  Dequantized value: scale16 * code + bias16.
* only the keys are rotated (y = R k, the rotation of the codebook path);
  values are quantized in their own frame, so the attention output needs no
  inverse rotation. The query is rotated into the keys' frame: <R q, y_hat>.
Everything is float64 apart from the fp16 storage of scale and bias.
"""

import math

import numpy as np

from .turboquant import rht, pack_codes, unpack_codes

__all__ = [
    "affine_levels", "affine_quantize_group_rows", "affine_dequant",
    "affine_code_ambiguous", "affine_encode_kv", "affine_attend",
    "affine_cache_bytes_per_token",
]


def affine_levels(bits: int) -> int:
    return (1 << bits) - 1


def _f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def affine_quantize_group_rows(y: np.ndarray, bits: int, group: int = 64):
    """y[..., d] -> (codes[..., d] uint8, scale16[..., d/group], bias16[..., d/group]).

    scale16 / bias16 are float64 arrays holding fp16 values."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    if d % group:
        raise ValueError("d must be a multiple of the group size")
    L = affine_levels(bits)
    yg = y.reshape(y.shape[:-1] + (d // group, group))
    lo = yg.min(axis=-1)
    hi = yg.max(axis=-1)
    scale = _f16((hi - lo) / L)
    bias = _f16(lo)
    s = scale[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s > 0, (yg - bias[..., None]) / np.where(s > 0, s, 1.0), 0.0)
    codes = np.clip(np.rint(u), 0, L).astype(np.uint8)
    return codes.reshape(y.shape), scale, bias


def affine_dequant(codes, scale16, bias16, group: int = 64) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.float64)
    d = codes.shape[-1]
    cg = codes.reshape(codes.shape[:-1] + (d // group, group))
    out = np.asarray(scale16)[..., None] * cg + np.asarray(bias16)[..., None]
    return out.reshape(codes.shape)


def affine_code_ambiguous(y, bits: int, group: int = 64, rel: float = 1e-9):
    """True where a code, a scale or a bias could flip under a relative
    perturbation of rel (different but equally exact summation orders of the
    rotation): (y - bias) / scale within rel of a half-integer, or the fp16
    rounding of the scale or bias within rel of a rounding boundary. Rows are
    flagged as a whole ([..., d] -> [...])."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    L = affine_levels(bits)
    yg = y.reshape(y.shape[:-1] + (d // group, group))
    lo = yg.min(axis=-1)
    hi = yg.max(axis=-1)
    raw_s = (hi - lo) / L

    def flips(v):
        return _f16(v * (1 - rel) - rel * 1e-30) != _f16(v * (1 + rel) + rel * 1e-30)

    bad = flips(raw_s) | flips(lo)
    codes, scale, bias = affine_quantize_group_rows(y, bits, group)
    s = scale[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s > 0, (yg - bias[..., None]) / np.where(s > 0, s, 1.0), 0.0)
    frac = np.abs(u - np.floor(u) - 0.5)
    near = (frac < rel * (1.0 + np.abs(u))) & (u > -0.5) & (u < L + 0.5)
    bad = bad | near.any(axis=-1)
    return bad.any(axis=-1)


def affine_encode_kv(k, v, *, bits_k, bits_v, seed, group: int = 64):
    """k, v: [..., d]. Returns a dict of packed planes in the library's layout:
    kc/vc [..., d*bits/8] uint8, ks/kb/vs/vb [..., d/group] fp16, plus the
    rotated keys ky (float64, for band checks)."""
    ky = rht(k, seed)
    kcodes, ks, kb = affine_quantize_group_rows(ky, bits_k, group)
    vcodes, vs, vb = affine_quantize_group_rows(np.asarray(v, np.float64), bits_v, group)
    return {
        "kc": pack_codes(kcodes, bits_k), "vc": pack_codes(vcodes, bits_v),
        "ks": ks.astype(np.float16), "kb": kb.astype(np.float16),
        "vs": vs.astype(np.float16), "vb": vb.astype(np.float16),
        "ky": ky,
    }


def affine_attend(q, cache, n_ctx, *, d, seed, bits_k, bits_v, Hkv, scale=None,
                  group: int = 64):
    """out[b, h] = sum_j softmax_j(tau <R q, y_hat_j>) v_hat_j over the first
    n_ctx tokens; query head h reads KV head h // (Hq / Hkv).

    q: [B][Hq][d]; cache planes [B][Hkv][capacity][...]. Returns [B][Hq][d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d) if not scale else scale
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for g in range(Hkv):
            ky = affine_dequant(unpack_codes(cache["kc"][b, g, :n_ctx], bits_k, d),
                                np.asarray(cache["ks"][b, g, :n_ctx], np.float64),
                                np.asarray(cache["kb"][b, g, :n_ctx], np.float64), group)
            vh = affine_dequant(unpack_codes(cache["vc"][b, g, :n_ctx], bits_v, d),
                                np.asarray(cache["vs"][b, g, :n_ctx], np.float64),
                                np.asarray(cache["vb"][b, g, :n_ctx], np.float64), group)
            for h in range(g * G, (g + 1) * G):
                s = tau * (ky @ rht(q[b, h], seed))
                p = np.exp(s - s.max())
                out[b, h] = (p @ vh) / p.sum()
    return out


def affine_cache_bytes_per_token(d: int, bits_k: int, bits_v: int, group: int = 64) -> int:
    """Bytes one token adds per KV head: codes plus fp16 scale and bias per group."""
    return d * (bits_k + bits_v) // 8 + 2 * (d // group) * 4
