"""TurboQuant KV-cache oracle: plain, slow, float64 NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring). Nothing in the product
path may import this module.

What the pages fix and what is a reading
----------------------------------------
The pages describe the method; they leave several encoding details open.
Each open detail below is marked READING and is the plainest choice that the
rest of the pages support.

* Rotation. Keys and values are rotated by a random Hadamard transform before
  quantization, and the query is rotated the same way ("What Is TurboQuant?"
  on the performance page; "What is TurboQuant?" on the API page, which names
  the helpers _rotation_matrix, _rht_forward, _rht_inverse; the README's
  introduction says the rotation is a randomized Hadamard transform and that
  it preserves inner products).
  READING: R = H_d diag(s) / sqrt(d) with H_d the Sylvester Hadamard matrix in
  natural order and s a +-1 vector from SplitMix64 (top output bit 1 -> -1).
* Codebook. An MSE codebook (performance page, "What Is TurboQuant?"; API
  page, `_codebook`; README: a non-uniform Lloyd-Max LUT). READING: the
  Lloyd-Max quantizer of N(0,1), applied to z = sqrt(d) * R x / ||x||.
* Code rule. READING: code_i = #{k : z_i >= t_k} (ties go up).
* Packing. Kernels work on packed data (performance page, "Custom Metal
  Kernel Implementation"); the README roadmap notes that 3-bit codes do not
  divide 32. READING: code i occupies bits [b*i, b*i+b) of the vector's
  little-endian byte string (a dense LSB-first bitstream).
* Norm. READING: one norm per vector, rounded to nearest-even into the norm
  dtype (fp16 or fp32); the decoder sees only the rounded norm.
* QJL residual (README, "The 1-bit QJL residual (unbiased inner-product
  estimator)"): r = R k - k_hat_rot, store sign(RHT_2(r)) and ||r||, estimate
  <Rq, r> by sqrt(pi/(2d)) ||r|| <RHT_2(Rq), sign(RHT_2(r))>.
  READING: "sqrt(pi/2d)" is sqrt(pi/(2d)); bit_i = 1 iff w_i < 0 (sign(0) = +1);
  bits packed LSB-first into 32-bit words (README, "The Metal kernels": the
  sign words are uint32); ||r|| stored as fp16.
* Fractional bits (performance page, "Fractional-Bit Precision Support"):
  3.5 bits means 3-bit keys and 4-bit values. READING: floor for keys, ceil
  for values for any non-integer width.
* GQA. READING: query head h uses KV head floor(h / G), G = Hq / Hkv.
"""

from __future__ import annotations

import functools
import math

import numpy as np

__all__ = [
    "MASK64", "splitmix64", "signs", "hadamard_sylvester", "fwht", "rht",
    "rht_inverse", "rotation_matrix", "lloyd_max", "codebook_mse",
    "quantize", "round_norm", "norm_ambiguous", "encode_vectors",
    "dequant_rot", "pack_codes", "unpack_codes", "pack_signs",
    "unpack_signs", "qjl_sketch", "qjl_from_encoding", "encode_kv",
    "attend", "attend_dense", "attend_rotated_blocked", "QJL_CONST",
    "turboquant_enabled", "bits_split", "tq_bytes_per_token",
    "affine_bytes_per_token", "fp16_bytes_per_token", "boundary_mask",
    "qjl_boundary_mask", "merge_partials", "attend_prefill", "sphere_density",
]

MASK64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# Seeded sign vector (API page, "What is TurboQuant?": a deterministic random
# rotation). The generator is SplitMix64 (Steele, Lea, Flood, "Fast
# splittable pseudorandom number generators", OOPSLA 2014).
# ---------------------------------------------------------------------------

def splitmix64(seed: int, n: int) -> list[int]:
    """First n outputs of SplitMix64 started from state `seed`."""
    state = seed & MASK64
    out = []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        out.append(z ^ (z >> 31))
    return out


def signs(seed: int, d: int) -> np.ndarray:
    """s_i = -1 if the top bit of the i-th SplitMix64 output is set, else +1."""
    return np.array([-1.0 if (w >> 63) else 1.0 for w in splitmix64(seed, d)])


# ---------------------------------------------------------------------------
# Randomized Hadamard transform (README introduction; API page helpers
# _rht_forward / _rht_inverse).
# ---------------------------------------------------------------------------

def hadamard_sylvester(d: int) -> np.ndarray:
    """Explicit Sylvester matrix: H_1 = [1], H_2m = [[H, H], [H, -H]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalized Walsh-Hadamard transform (H_d x) along the last axis.

    Butterflies on index bit 0, 1, ..., log2(d)-1; equals H_d @ x for the
    Sylvester H_d.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    lead = x.shape[:-1]
    h = 1
    while h < d:
        y = x.reshape(lead + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        x = y.reshape(lead + (d,))
        h *= 2
    return x


def rht(x: np.ndarray, seed: int) -> np.ndarray:
    """R x with R = H_d diag(s) / sqrt(d): sign flip, then normalized WHT."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return fwht(x * signs(seed, d)) / math.sqrt(d)


def rht_inverse(y: np.ndarray, seed: int) -> np.ndarray:
    """R^T y = diag(s) H_d y / sqrt(d) (R is orthogonal, H_d symmetric)."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    return signs(seed, d) * fwht(y) / math.sqrt(d)


def rotation_matrix(seed: int, d: int) -> np.ndarray:
    """Dense R, for tiny-d brute-force checks only."""
    return hadamard_sylvester(d) * signs(seed, d)[None, :] / math.sqrt(d)


# ---------------------------------------------------------------------------
# Lloyd-Max codebook for N(0,1) (performance page "What Is TurboQuant?": MSE
# code-book; README: non-uniform Lloyd-Max LUT; README introduction: the
# rotated marginal is near-Gaussian).
# ---------------------------------------------------------------------------

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi(x: float) -> float:
    return 0.0 if math.isinf(x) else _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _upper_tail(x: float) -> float:
    """P(Z >= x) for x >= 0, without cancellation."""
    return 0.0 if math.isinf(x) else 0.5 * math.erfc(x / _SQRT2)


def _cell_mean(a: float, b: float) -> float:
    """E[Z | a <= Z < b] for 0 <= a < b <= inf."""
    return (_phi(a) - _phi(b)) / (_upper_tail(a) - _upper_tail(b))


def lloyd_max(bits: int, sphere_d: int | None = None):
    """Centroids (ascending, 2^bits) and thresholds (2^bits - 1) in float64.

    Lloyd iteration on the positive half-line, then mirrored, so the codebook
    is exactly antisymmetric and the middle threshold is exactly 0.
    sphere_d=None: the quantizer of N(0,1), the near-Gaussian marginal the
    pages name. sphere_d=d: the quantizer of the exact finite-d marginal of
    z = sqrt(d) u, u one coordinate of a uniformly random unit vector in R^d
    (density proportional to (1 - z^2/d)^((d-3)/2) on |z| < sqrt(d)); the
    roadmap variant for small head dimensions.
    """
    c, t = _lloyd_max_cached(bits) if sphere_d is None else _sphere_lloyd_cached(bits, sphere_d)
    return np.array(c), np.array(t)


def sphere_density(z, d: int):
    """Unnormalized density of z = sqrt(d) u for u a coordinate of a uniform
    unit vector in R^d: (1 - z^2/d)^((d-3)/2) on |z| < sqrt(d)."""
    z = np.asarray(z, dtype=np.float64)
    inside = np.abs(z) < math.sqrt(d)
    return np.where(inside, np.clip(1.0 - z * z / d, 0.0, None) ** ((d - 3) / 2.0), 0.0)


@functools.lru_cache(maxsize=None)
def _sphere_lloyd_cached(bits: int, d: int, tol: float = 1e-13, max_iter: int = 100000):
    import scipy.integrate
    if bits < 1 or d < 4:
        raise ValueError("bits >= 1 and d >= 4")
    m = 1 << (bits - 1)
    k = (d - 3) / 2.0
    zmax = math.sqrt(d)

    def base(z):
        return max(0.0, 1.0 - z * z / d)   # 0 at the end point sqrt(d)

    def mass(a, b):
        return scipy.integrate.quad(lambda z: base(z) ** k, a, b,
                                    epsabs=1e-300, epsrel=1e-13, limit=400)[0]

    def first(a, b):
        # integral of z (1 - z^2/d)^k, in closed form
        return d / (2.0 * (k + 1.0)) * (base(a) ** (k + 1.0) - base(b) ** (k + 1.0))

    c = [min(v, 0.9 * zmax) for v in _lloyd_max_cached(bits)[0][m:]]
    for _ in range(max_iter):
        edges = [0.0] + [(c[i - 1] + c[i]) / 2.0 for i in range(1, m)] + [zmax]
        new = [first(edges[i], edges[i + 1]) / mass(edges[i], edges[i + 1]) for i in range(m)]
        delta = max(abs(u - v) for u, v in zip(new, c))
        c = new
        if delta < tol:
            break
    pos = list(c)
    inner = [(pos[i - 1] + pos[i]) / 2.0 for i in range(1, m)]
    centroids = [-v for v in reversed(pos)] + pos
    thresholds = [-v for v in reversed(inner)] + [0.0] + inner
    return tuple(centroids), tuple(thresholds)


@functools.lru_cache(maxsize=None)
def _lloyd_max_cached(bits: int, tol: float = 1e-15, max_iter: int = 200000):
    if bits < 1:
        raise ValueError("bits must be >= 1")
    m = 1 << (bits - 1)                    # levels on the positive side
    # start from equal-probability cells of the half-normal
    c = [math.sqrt(2.0) * _erfinv((k + 0.5) / m) for k in range(m)]
    for _ in range(max_iter):
        edges = [0.0] + [(c[k - 1] + c[k]) / 2.0 for k in range(1, m)] + [math.inf]
        new = [_cell_mean(edges[k], edges[k + 1]) for k in range(m)]
        delta = max(abs(u - v) for u, v in zip(new, c))
        c = new
        if delta < tol:
            break
    pos = list(c)
    inner = [(pos[k - 1] + pos[k]) / 2.0 for k in range(1, m)]
    centroids = [-v for v in reversed(pos)] + pos
    thresholds = [-v for v in reversed(inner)] + [0.0] + inner
    return tuple(centroids), tuple(thresholds)


def _erfinv(y: float) -> float:
    """Inverse error function by bisection (only seeds the Lloyd iteration)."""
    lo, hi = 0.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if math.erf(mid) < y:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def codebook_mse(bits: int) -> float:
    """E[(Z - Q(Z))^2] for the Lloyd-Max quantizer, cell by cell."""
    c, t = lloyd_max(bits)
    edges = [-math.inf] + list(t) + [math.inf]
    total = 0.0
    for k, ck in enumerate(c):
        a, b = edges[k], edges[k + 1]
        # integral of (z - ck)^2 phi(z) over [a, b):
        #   second moment - 2 ck first moment + ck^2 mass
        mass = _mass(a, b)
        first = _phi(a) - _phi(b)
        second = mass + (a * _phi(a) if not math.isinf(a) else 0.0) \
            - (b * _phi(b) if not math.isinf(b) else 0.0)
        total += second - 2.0 * ck * first + ck * ck * mass
    return total


def _mass(a: float, b: float) -> float:
    """P(a <= Z < b) for any a < b."""
    if a >= 0:
        return _upper_tail(a) - _upper_tail(b)
    if b <= 0:
        return _upper_tail(-b) - _upper_tail(-a)
    return 1.0 - _upper_tail(-a) - _upper_tail(b)


def quantize(z: np.ndarray, thresholds: np.ndarray) -> np.ndarray:
    """code = #{k : z >= t_k}; a value equal to a threshold goes up."""
    z = np.asarray(z, dtype=np.float64)
    return (z[..., None] >= thresholds).sum(axis=-1).astype(np.uint8)


def boundary_mask(z: np.ndarray, thresholds: np.ndarray, eps: float = 1e-6):
    """True where z lies within eps of a decision threshold (either code ok)."""
    z = np.asarray(z, dtype=np.float64)
    return (np.abs(z[..., None] - thresholds) < eps).any(axis=-1)


# ---------------------------------------------------------------------------
# Per-vector norm (READING: one norm per vector, nearest-even rounding).
# ---------------------------------------------------------------------------

_NORM_TYPES = {"f16": np.float16, "f32": np.float32}


def round_norm(n: np.ndarray, norm_dtype: str) -> np.ndarray:
    """Round a float64 norm to nearest-even in the norm dtype, back to f64."""
    return np.asarray(n, dtype=np.float64).astype(_NORM_TYPES[norm_dtype]).astype(np.float64)


def norm_ambiguous(n: np.ndarray, norm_dtype: str, rel: float = 1e-6):
    """True where n is within rel of a rounding midpoint of the norm dtype."""
    n = np.asarray(n, dtype=np.float64)
    return round_norm(n * (1 - rel), norm_dtype) != round_norm(n * (1 + rel), norm_dtype)


# ---------------------------------------------------------------------------
# Encode (performance page "What Is TurboQuant?": rotation then MSE codebook).
# ---------------------------------------------------------------------------

def encode_vectors(x: np.ndarray, seed: int, bits: int, norm_dtype: str, sphere: bool = False):
    """Encode rows x[..., d].

    Returns dict with codes (uint8, ascending-codebook indices), norm (rounded,
    float64), norm_exact (float64), z (float64 scaled rotated coordinates),
    y (= R x).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    _, thr = lloyd_max(bits, x.shape[-1] if sphere else None)
    n = np.sqrt((x * x).sum(axis=-1))
    y = rht(x, seed)
    safe = np.where(n > 0, n, 1.0)
    z = np.where((n > 0)[..., None], math.sqrt(d) * y / safe[..., None], 0.0)
    return {
        "codes": quantize(z, thr),
        "norm": round_norm(n, norm_dtype),
        "norm_exact": n,
        "z": z,
        "y": y,
    }


def dequant_rot(codes: np.ndarray, norm: np.ndarray, bits: int,
                sphere: bool = False) -> np.ndarray:
    """x_hat in the rotated frame: norm * c[code] / sqrt(d)."""
    c, _ = lloyd_max(bits, np.shape(codes)[-1] if sphere else None)
    codes = np.asarray(codes)
    d = codes.shape[-1]
    return np.asarray(norm, dtype=np.float64)[..., None] * c[codes] / math.sqrt(d)


# ---------------------------------------------------------------------------
# Bit packing (READING: dense LSB-first bitstream per vector).
# ---------------------------------------------------------------------------

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes[..., d] -> bytes[..., d*bits/8]; code i at bits [bits*i, bits*i+bits)."""
    codes = np.asarray(codes, dtype=np.uint8)
    d = codes.shape[-1]
    if (d * bits) % 8:
        raise ValueError("d*bits must be a multiple of 8")
    planes = (codes[..., :, None] >> np.arange(bits, dtype=np.uint8)) & 1
    stream = planes.reshape(codes.shape[:-1] + (d * bits,))
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack_codes(packed: np.ndarray, bits: int, d: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    stream = np.unpackbits(packed, axis=-1, bitorder="little")
    stream = stream.reshape(packed.shape[:-1] + (d, bits)).astype(np.uint8)
    return (stream << np.arange(bits, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)


def pack_signs(bits01: np.ndarray) -> np.ndarray:
    """bits[..., d] (0/1) -> bytes[..., d/8], LSB-first; the same bytes read as
    little-endian uint32 words put coordinate 32m + j at bit j of word m."""
    return np.packbits(np.asarray(bits01, dtype=np.uint8), axis=-1, bitorder="little")


def unpack_signs(packed: np.ndarray, d: int) -> np.ndarray:
    return np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=-1,
                         bitorder="little")[..., :d]


# ---------------------------------------------------------------------------
# QJL residual sketch (README, "The 1-bit QJL residual").
# ---------------------------------------------------------------------------

QJL_CONST = math.pi / 2.0   # the estimator's factor is sqrt(QJL_CONST / d)


def qjl_sketch(r: np.ndarray, qjl_seed: int):
    """sign bits of R_2 r (1 where negative) and ||r|| rounded to fp16."""
    r = np.asarray(r, dtype=np.float64)
    w = rht(r, qjl_seed)
    bits01 = (w < 0).astype(np.uint8)
    rnorm_exact = np.sqrt((r * r).sum(axis=-1))
    return {
        "bits": bits01,
        "packed": pack_signs(bits01),
        "rnorm": round_norm(rnorm_exact, "f16"),
        "rnorm_exact": rnorm_exact,
        "w": w,
    }


def qjl_boundary_mask(w: np.ndarray, rnorm_exact: np.ndarray, rel: float = 1e-6):
    """True where |w_i| < rel * ||r|| (either sign bit acceptable)."""
    return np.abs(w) < rel * np.asarray(rnorm_exact)[..., None]


def qjl_from_encoding(enc: dict, bits: int, qjl_seed: int, sphere: bool = False):
    """Residual of an encoded key in the rotated frame, then its sketch.

    r = R k - k_hat_rot with k_hat_rot built from the STORED (rounded) norm.
    """
    r = enc["y"] - dequant_rot(enc["codes"], enc["norm"], bits, sphere)
    out = qjl_sketch(r, qjl_seed)
    out["r"] = r
    return out


# ---------------------------------------------------------------------------
# Whole-cache encode: planes laid out [B][Hkv][n][bytes].
# ---------------------------------------------------------------------------

def encode_kv(k, v, *, seed, bits_k, bits_v, norm_dtype, qjl=False, qjl_seed=None,
              sphere=False):
    """Encode K and V rows [B][Hkv][n][d] into packed planes (numpy arrays).
    sphere: use the finite-d marginal codebook (lloyd_max(bits, d))."""
    ek = encode_vectors(k, seed, bits_k, norm_dtype, sphere)
    ev = encode_vectors(v, seed, bits_v, norm_dtype, sphere)
    out = {
        "kc": pack_codes(ek["codes"], bits_k),
        "vc": pack_codes(ev["codes"], bits_v),
        "kn": ek["norm"], "vn": ev["norm"],
        "k_enc": ek, "v_enc": ev,
    }
    if qjl:
        sk = qjl_from_encoding(ek, bits_k, seed + 1 if qjl_seed is None else qjl_seed, sphere)
        out["kq"] = sk["packed"]
        out["kr"] = sk["rnorm"]
        out["k_qjl"] = sk
    return out


# ---------------------------------------------------------------------------
# Decode attention (performance page, "Custom Metal Kernel Implementation":
# scores on packed codes fused with value aggregation; README "How it plugs
# in": the query is rotated, and the QJL correction is added to the score).
# ---------------------------------------------------------------------------

def _scores_rot(qr, kcodes, knorm, bits_k, tau, qjl=None, sphere=False):
    """tau * <R q, k_hat_rot> (+ QJL term), qr = R q [Hg][d] -> [Hg][n]."""
    khat = dequant_rot(kcodes, knorm, bits_k, sphere)    # [n][d]
    s = qr @ khat.T
    if qjl is not None:
        qq, sigma, rnorm = qjl                           # qq = R2 R q [Hg][d]
        d = qr.shape[-1]
        s = s + math.sqrt(QJL_CONST / d) * (qq @ sigma.T) * rnorm[None, :]
    return tau * s


def attend_dense(q, cache, *, d, seed, bits_k, bits_v, Hkv, scale=None,
                 qjl=False, qjl_seed=None, sphere=False):
    """Dense mode: dequantize K and V to the original frame, then
    softmax(q K_hat^T tau [+ QJL]) V_hat in float64.

    q: [B][Hq][d]; cache planes as produced by encode_kv (possibly sliced to
    the first n_ctx tokens). Returns [B][Hq][d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d) if not scale else scale
    qs = seed + 1 if qjl_seed is None else qjl_seed
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for g in range(Hkv):
            kc = unpack_codes(cache["kc"][b, g], bits_k, d)
            vc = unpack_codes(cache["vc"][b, g], bits_v, d)
            k_hat = rht_inverse(dequant_rot(kc, cache["kn"][b, g], bits_k, sphere), seed)
            v_hat = rht_inverse(dequant_rot(vc, cache["vn"][b, g], bits_v, sphere), seed)
            qh = q[b, g * G:(g + 1) * G]                 # [G][d]
            logits = tau * (qh @ k_hat.T)
            if qjl:
                sigma = 1.0 - 2.0 * unpack_signs(cache["kq"][b, g], d)
                qq = rht(rht(qh, seed), qs)
                logits = logits + tau * math.sqrt(QJL_CONST / d) * \
                    (qq @ sigma.T) * cache["kr"][b, g][None, :]
            logits = logits - logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            out[b, g * G:(g + 1) * G] = p @ v_hat
    return out


def merge_partials(ms, ls, accs):
    """Exact log-sum-exp merge of (max, sum, weighted-sum) partials."""
    ms = np.asarray(ms)
    M = ms.max()
    w = np.exp(ms - M)
    return (w[:, None] * np.asarray(accs)).sum(axis=0) / (w * np.asarray(ls)).sum()


def attend_rotated_blocked(q, kv_block_fn, n_ctx, *, B, Hq, Hkv, d, seed,
                           bits_k, bits_v, scale=None, qjl=False,
                           qjl_seed=None, block=65536, heads=None, sphere=False):
    """Rotated-frame mode for long contexts.

    kv_block_fn(b, g, t0, t1) returns a dict with unpacked arrays for tokens
    [t0, t1): kcodes, kn, vcodes, vn (+ ksig (0/1 bits), kr when qjl).
    Scores and values stay in the rotated frame; blocks are merged with an
    exact log-sum-exp; the output is rotated back once per query head.
    heads: optional list of (b, h) query heads to compute (others left 0).
    """
    q = np.asarray(q, dtype=np.float64)
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d) if not scale else scale
    qs = seed + 1 if qjl_seed is None else qjl_seed
    want = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    groups = {}
    for (b, h) in want:
        groups.setdefault((b, h // G), []).append(h)
    out = np.zeros((B, Hq, d))
    for (b, g), hs in groups.items():
        qr = rht(q[b, hs], seed)                          # [nh][d]
        qq = rht(qr, qs) if qjl else None
        ms, ls, accs = [], [], []
        for t0 in range(0, n_ctx, block):
            t1 = min(n_ctx, t0 + block)
            blk = kv_block_fn(b, g, t0, t1)
            qj = None
            if qjl:
                qj = (qq, 1.0 - 2.0 * blk["ksig"].astype(np.float64), blk["kr"])
            lg = _scores_rot(qr, blk["kcodes"], blk["kn"], bits_k, tau, qj, sphere)
            m = lg.max(axis=1)
            p = np.exp(lg - m[:, None])
            vhat = dequant_rot(blk["vcodes"], blk["vn"], bits_v, sphere)
            ms.append(m)
            ls.append(p.sum(axis=1))
            accs.append(p @ vhat)
        ms, ls, accs = np.array(ms), np.array(ls), np.array(accs)
        for i, h in enumerate(hs):
            orot = merge_partials(ms[:, i], ls[:, i], accs[:, i])
            out[b, h] = rht_inverse(orot, seed)
    return out


def attend(q, cache, n_ctx, *, d, seed, bits_k, bits_v, Hkv, scale=None,
           qjl=False, qjl_seed=None, block=65536, sphere=False):
    """Rotated-blocked attention over an in-memory cache (first n_ctx tokens)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, _ = q.shape

    def fn(b, g, t0, t1):
        blk = {
            "kcodes": unpack_codes(cache["kc"][b, g, t0:t1], bits_k, d),
            "kn": np.asarray(cache["kn"][b, g, t0:t1], dtype=np.float64),
            "vcodes": unpack_codes(cache["vc"][b, g, t0:t1], bits_v, d),
            "vn": np.asarray(cache["vn"][b, g, t0:t1], dtype=np.float64),
        }
        if qjl:
            blk["ksig"] = unpack_signs(cache["kq"][b, g, t0:t1], d)
            blk["kr"] = np.asarray(cache["kr"][b, g, t0:t1], dtype=np.float64)
        return blk

    return attend_rotated_blocked(q, fn, n_ctx, B=B, Hq=Hq, Hkv=Hkv, d=d,
                                  seed=seed, bits_k=bits_k, bits_v=bits_v,
                                  scale=scale, qjl=qjl, qjl_seed=qjl_seed,
                                  block=block, sphere=sphere)


def attend_prefill(q, cache, n_ctx, *, d, seed, bits_k, bits_v, Hkv, scale=None,
                   qjl=False, qjl_seed=None, sphere=False):
    """Causal multi-query attention of a prefill chunk over the packed cache.

    The chunk's n_q tokens are the last n_q of the first n_ctx cache rows
    (they were appended before the call); query i sits at position
    p_i = n_ctx - n_q + i and attends to tokens 0..p_i. This is the same
    score, softmax and value sum as `attend_dense` (the API page's patched
    attention: the query rotated into the cache's frame, the QJL term added),
    with the causal mask of a prefill step.

    q: [B][Hq][n_q][d]. Returns [B][Hq][n_q][d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, n_q, _ = q.shape
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d) if not scale else scale
    qs = seed + 1 if qjl_seed is None else qjl_seed
    pos = n_ctx - n_q + np.arange(n_q)
    future = np.arange(n_ctx)[None, :] > pos[:, None]         # [n_q][n_ctx]
    out = np.zeros((B, Hq, n_q, d))
    for b in range(B):
        for g in range(Hkv):
            kc = unpack_codes(cache["kc"][b, g, :n_ctx], bits_k, d)
            vc = unpack_codes(cache["vc"][b, g, :n_ctx], bits_v, d)
            k_hat = rht_inverse(dequant_rot(kc, cache["kn"][b, g, :n_ctx], bits_k, sphere), seed)
            v_hat = rht_inverse(dequant_rot(vc, cache["vn"][b, g, :n_ctx], bits_v, sphere), seed)
            if qjl:
                sigma = 1.0 - 2.0 * unpack_signs(cache["kq"][b, g, :n_ctx], d)
            for h in range(g * G, (g + 1) * G):
                logits = tau * (q[b, h] @ k_hat.T)                 # [n_q][n_ctx]
                if qjl:
                    qq = rht(rht(q[b, h], seed), qs)
                    logits = logits + tau * math.sqrt(QJL_CONST / d) * \
                        (qq @ sigma.T) * cache["kr"][b, g, :n_ctx][None, :]
                logits = np.where(future, -np.inf, logits)
                logits = logits - logits.max(axis=1, keepdims=True)
                p = np.exp(logits)
                p /= p.sum(axis=1, keepdims=True)
                out[b, h] = p @ v_hat
    return out


# ---------------------------------------------------------------------------
# Enable rule and fractional split (API page, "How TurboQuant Activation
# Works"; performance page, "Fractional-Bit Precision Support").
# ---------------------------------------------------------------------------

def turboquant_enabled(kv_bits, scheme=None) -> bool:
    """Off without a bit width; on when forced by scheme, else on exactly
    when the width is farther than 1e-6 from the nearest integer."""
    if kv_bits is None:
        return False
    if scheme == "turboquant":
        return True
    kv_bits = float(kv_bits)
    return abs(kv_bits - round(kv_bits)) > 1e-6


def bits_split(kv_bits, scheme=None):
    """(bits_k, bits_v) or None when TurboQuant is not selected.

    Non-integer widths: keys take the floor, values the ceiling (3.5 -> 3/4 is
    fixed by the pages; others are a READING). Integer widths (forced by the
    scheme) use the same width for both.
    """
    if not turboquant_enabled(kv_bits, scheme):
        return None
    kv_bits = float(kv_bits)
    r = round(kv_bits)
    if abs(kv_bits - r) <= 1e-6:
        return int(r), int(r)
    return int(math.floor(kv_bits)), int(math.ceil(kv_bits))


# ---------------------------------------------------------------------------
# Byte accounting (README, "Memory footprint over long context").
# ---------------------------------------------------------------------------

def tq_bytes_per_token(d, bits_k, bits_v, norm_bytes, qjl, n_kv_vectors=1):
    """Bytes per token of this format for n_kv_vectors (layers x KV heads)."""
    per = d * bits_k // 8 + norm_bytes + d * bits_v // 8 + norm_bytes
    if qjl:
        per += d // 8 + 2            # sign bits + fp16 residual norm
    return per * n_kv_vectors


def affine_bytes_per_token(elems_per_token_kv, bits, group=64, qjl_d=None):
    """Group-affine KV (fp16 scale and bias per group) as the README measures
    it; elems_per_token_kv counts K plus V elements. qjl_d: add a 1-bit sketch
    of the keys plus one fp16 residual norm per key vector of that length."""
    total = elems_per_token_kv * bits / 8 + (elems_per_token_kv // group) * 4
    if qjl_d:
        keys = elems_per_token_kv // 2
        total += keys / 8 + (keys // qjl_d) * 2
    return total


def fp16_bytes_per_token(elems_per_token_kv):
    return 2 * elems_per_token_kv
