"""ctypes binding of libtq.so: the same entry points as include/tq.h.

Argument marshalling only. Every computation runs in the HIP kernels of
libtq.so; torch is used for device memory and streams. Loading fails loudly
when libtq.so is missing (build it with `python -m
decode_attention_seeded_amd.build`); there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK = 0
TQ_ERR_ARG = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_ALIGN = -3
TQ_ERR_CAPACITY = -4
TQ_ERR_WORKSPACE = -5
TQ_ERR_NO_DEVICE = -6
TQ_ERR_HIP = -7

TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_CODEBOOK_GAUSS, TQ_CODEBOOK_SPHERE = 0, 1

# every symbol include/tq.h declares
EXPORTS = (
    "tq_bits_split", "tq_codebook", "tq_codebook_ex", "tq_signs", "tq_cache_bytes", "tq_rht",
    "tq_encode_kv", "tq_qjl_sketch", "tq_num_splits", "tq_workspace_bytes",
    "tq_attend_decode", "tq_attend_decode_noalloc", "tq_append_attend_decode",
    "tq_append_chunk_attend_decode", "tq_dense_workspace_bytes",
    "tq_dense_decode_bf16", "tq_attend_prefill", "tq_read_probe_sink_words",
    "tq_read_probe", "tq_affine_cache_bytes", "tq_affine_encode_kv", "tq_affine_num_splits",
    "tq_affine_workspace_bytes", "tq_affine_attend_decode",
    "tq_strerror",
)


class TqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib().tq_strerror(status).decode()} ({status})")


class tq_config(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("bits_k", ctypes.c_int), ("bits_v", ctypes.c_int),
                ("norm_dtype", ctypes.c_int), ("qjl", ctypes.c_int),
                ("seed", ctypes.c_uint64), ("qjl_seed", ctypes.c_uint64),
                ("codebook", ctypes.c_int)]


class tq_cache(ctypes.Structure):
    _fields_ = [("kc", ctypes.c_void_p), ("vc", ctypes.c_void_p), ("kn", ctypes.c_void_p),
                ("vn", ctypes.c_void_p), ("kq", ctypes.c_void_p), ("kr", ctypes.c_void_p),
                ("B", ctypes.c_int), ("Hkv", ctypes.c_int), ("capacity", ctypes.c_int64)]


class tq_affine_config(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("bits_k", ctypes.c_int), ("bits_v", ctypes.c_int),
                ("group", ctypes.c_int), ("seed", ctypes.c_uint64)]


class tq_affine_cache(ctypes.Structure):
    _fields_ = [("kc", ctypes.c_void_p), ("vc", ctypes.c_void_p), ("ks", ctypes.c_void_p),
                ("kb", ctypes.c_void_p), ("vs", ctypes.c_void_p), ("vb", ctypes.c_void_p),
                ("B", ctypes.c_int), ("Hkv", ctypes.c_int), ("capacity", ctypes.c_int64)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library with "
                "`python -m decode_attention_seeded_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, I64, U64, F, D, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_uint64, ctypes.c_float, ctypes.c_double,
                                    ctypes.c_size_t)
        CFG, CACHE = ctypes.POINTER(tq_config), ctypes.POINTER(tq_cache)
        ACFG, ACACHE = ctypes.POINTER(tq_affine_config), ctypes.POINTER(tq_affine_cache)
        sig = {
            "tq_bits_split": (I, [D, I, ctypes.POINTER(I), ctypes.POINTER(I), ctypes.POINTER(I)]),
            "tq_codebook": (I, [I, P, P]),
            "tq_codebook_ex": (I, [I, I, I, P, P]),
            "tq_signs": (I, [U64, I, P]),
            "tq_cache_bytes": (I64, [CFG, I, I, I64, P]),
            "tq_rht": (I, [P, I, P, I64, I, U64, I, P]),
            "tq_encode_kv": (I, [CFG, P, P, I, I64, I64, CACHE, P]),
            "tq_qjl_sketch": (I, [P, I64, I, U64, P, P, P]),
            "tq_num_splits": (I, [CFG, I, I, I, I64, I]),
            "tq_workspace_bytes": (I64, [CFG, I, I, I, I64, I]),
            "tq_attend_decode": (I, [CFG, P, I, I, I, CACHE, I64, F, I, P, P, SZ, P]),
            "tq_attend_decode_noalloc": (I, [CFG, P, I, I, I, CACHE, I64, F, I, P, P]),
            "tq_append_attend_decode": (I, [CFG, P, P, I, P, I, I, I, CACHE, I64, F, I, P, P,
                                            SZ, P]),
            "tq_append_chunk_attend_decode": (I, [CFG, P, P, I, I64, P, I, I, I, CACHE, I64,
                                                  F, I, P, P, SZ, P]),
            "tq_dense_workspace_bytes": (I64, [I, I, I, I, I64, I]),
            "tq_dense_decode_bf16": (I, [P, P, P, I, I, I, I, I64, F, I, P, P, SZ, P]),
            "tq_attend_prefill": (I, [CFG, P, I, I, I, I64, CACHE, I64, F, P, P]),
            "tq_read_probe_sink_words": (I64, [I64]),
            "tq_read_probe": (I, [P, I64, P, P]),
            "tq_affine_cache_bytes": (I64, [ACFG, I, I, I64, P]),
            "tq_affine_encode_kv": (I, [ACFG, P, P, I, I64, I64, ACACHE, P]),
            "tq_affine_num_splits": (I, [ACFG, I, I, I, I64, I]),
            "tq_affine_workspace_bytes": (I64, [ACFG, I, I, I, I64, I]),
            "tq_affine_attend_decode": (I, [ACFG, P, I, I, I, ACACHE, I64, F, I, P, P, SZ, P]),
            "tq_strerror": (ctypes.c_char_p, [I]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def lib():
    """The loaded libtq.so (raises ImportError when it was not built)."""
    return _lib()


def _check(status, where):
    if status < 0:
        raise TqError(int(status), where)
    return status


# ---------------------------------------------------------------------------
# Python-level description of a format
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    d: int = 128
    bits_k: int = 3
    bits_v: int = 4
    norm_dtype: str = "f16"       # "f16" | "f32"
    qjl: bool = False
    seed: int = 0
    qjl_seed: int = 1
    codebook: str = "gauss"       # "gauss" | "sphere" (exact finite-d marginal)

    def c(self) -> tq_config:
        return tq_config(self.d, self.bits_k, self.bits_v,
                         TQ_F16 if self.norm_dtype == "f16" else TQ_F32,
                         int(self.qjl), self.seed, self.qjl_seed,
                         TQ_CODEBOOK_SPHERE if self.codebook == "sphere" else TQ_CODEBOOK_GAUSS)


def _dtype_code(t):
    import torch
    m = {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}
    if t.dtype not in m:
        raise TqError(TQ_ERR_UNSUPPORTED, f"dtype {t.dtype}")
    return m[t.dtype]


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# ---------------------------------------------------------------------------
# Host-only entry points
# ---------------------------------------------------------------------------

def tq_strerror(status: int) -> str:
    return _lib().tq_strerror(status).decode()


def tq_bits_split(kv_bits: float, force_turboquant: bool = False):
    """(bits_k, bits_v), or None when TurboQuant is not selected."""
    en, bk, bv = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(_lib().tq_bits_split(float(kv_bits), int(force_turboquant), ctypes.byref(en),
                                ctypes.byref(bk), ctypes.byref(bv)), "tq_bits_split")
    return (bk.value, bv.value) if en.value else None


def tq_codebook(bits: int):
    """(centroids, thresholds) as Python float lists (double precision)."""
    L = 1 << bits
    c = (ctypes.c_double * L)()
    t = (ctypes.c_double * max(L - 1, 1))()
    _check(_lib().tq_codebook(bits, ctypes.cast(c, ctypes.c_void_p),
                              ctypes.cast(t, ctypes.c_void_p)), "tq_codebook")
    return list(c), list(t)[:L - 1]


def tq_codebook_ex(bits: int, kind: str = "gauss", d: int = 128):
    """The codebook a config selects ("gauss" or "sphere" at head dim d), as
    (centroids, thresholds) Python float lists."""
    L = 1 << bits
    c = (ctypes.c_double * L)()
    t = (ctypes.c_double * max(L - 1, 1))()
    k = TQ_CODEBOOK_SPHERE if kind == "sphere" else TQ_CODEBOOK_GAUSS
    _check(_lib().tq_codebook_ex(bits, k, d, ctypes.cast(c, ctypes.c_void_p),
                                 ctypes.cast(t, ctypes.c_void_p)), "tq_codebook_ex")
    return list(c), list(t)[:L - 1]


def tq_signs(seed: int, d: int):
    out = (ctypes.c_int8 * d)()
    _check(_lib().tq_signs(seed, d, ctypes.cast(out, ctypes.c_void_p)), "tq_signs")
    return list(out)


def tq_cache_bytes(cfg: Config, B: int, Hkv: int, capacity: int):
    planes = (ctypes.c_int64 * 6)()
    total = _check(_lib().tq_cache_bytes(ctypes.byref(cfg.c()), B, Hkv, capacity,
                                         ctypes.cast(planes, ctypes.c_void_p)), "tq_cache_bytes")
    return total, list(planes)


def tq_num_splits(cfg: Config, B, Hq, Hkv, n_ctx, splits=0):
    return _check(_lib().tq_num_splits(ctypes.byref(cfg.c()), B, Hq, Hkv, n_ctx, splits),
                  "tq_num_splits")


def tq_workspace_bytes(cfg: Config, B, Hq, Hkv, n_ctx, splits=0):
    return _check(_lib().tq_workspace_bytes(ctypes.byref(cfg.c()), B, Hq, Hkv, n_ctx, splits),
                  "tq_workspace_bytes")


def tq_dense_workspace_bytes(B, Hq, Hkv, d, n_ctx, splits=0):
    return _check(_lib().tq_dense_workspace_bytes(B, Hq, Hkv, d, n_ctx, splits),
                  "tq_dense_workspace_bytes")


# ---------------------------------------------------------------------------
# Packed cache: caller-owned device planes (torch tensors)
# ---------------------------------------------------------------------------

class PackedCache:
    """Device planes of a packed cache [B][Hkv][capacity]; see tq_cache in tq.h."""

    def __init__(self, cfg: Config, B: int, Hkv: int, capacity: int, device="cuda"):
        import torch
        self.cfg, self.B, self.Hkv, self.capacity = cfg, B, Hkv, capacity
        _, p = tq_cache_bytes(cfg, B, Hkv, capacity)
        shape = (B, Hkv, capacity)
        u8 = dict(dtype=torch.uint8, device=device)
        self.kc = torch.empty(shape + (cfg.d * cfg.bits_k // 8,), **u8)
        self.vc = torch.empty(shape + (cfg.d * cfg.bits_v // 8,), **u8)
        nd = torch.float16 if cfg.norm_dtype == "f16" else torch.float32
        self.kn = torch.empty(shape, dtype=nd, device=device)
        self.vn = torch.empty(shape, dtype=nd, device=device)
        self.kq = torch.empty(shape + (cfg.d // 8,), **u8) if cfg.qjl else None
        self.kr = torch.empty(shape, dtype=torch.float16, device=device) if cfg.qjl else None
        assert self.kc.numel() == p[0] and self.vc.numel() == p[1]

    def c(self) -> tq_cache:
        return tq_cache(self.kc.data_ptr(), self.vc.data_ptr(), self.kn.data_ptr(),
                        self.vn.data_ptr(),
                        self.kq.data_ptr() if self.kq is not None else None,
                        self.kr.data_ptr() if self.kr is not None else None,
                        self.B, self.Hkv, self.capacity)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in
                   (self.kc, self.vc, self.kn, self.vn, self.kq, self.kr) if t is not None)


# ---------------------------------------------------------------------------
# Device entry points
# ---------------------------------------------------------------------------

def tq_rht(x, y, seed: int = 0, inverse: bool = False, stream=None):
    """y[rows][d] (fp32) = R x or R^T x."""
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    _check(_lib().tq_rht(_ptr(x), _dtype_code(x), _ptr(y), rows, d, seed, int(inverse),
                         _stream(stream)), "tq_rht")


def tq_encode_kv(cfg: Config, k, v, offset: int, cache: PackedCache, stream=None):
    """Encode k, v [B][Hkv][n_new][d] at token positions [offset, offset+n_new)."""
    if k.shape != v.shape or k.dtype != v.dtype:
        raise TqError(TQ_ERR_ARG, "tq_encode_kv: k and v differ in shape or dtype")
    if k.dim() != 4 or k.shape[0] != cache.B or k.shape[1] != cache.Hkv or k.shape[3] != cfg.d:
        raise TqError(TQ_ERR_ARG, "tq_encode_kv: k must be [B][Hkv][n_new][d]")
    if not (k.is_contiguous() and v.is_contiguous()):
        raise TqError(TQ_ERR_ARG, "tq_encode_kv: k and v must be contiguous")
    c = cache.c()
    _check(_lib().tq_encode_kv(ctypes.byref(cfg.c()), _ptr(k), _ptr(v), _dtype_code(k), offset,
                               k.shape[2], ctypes.byref(c), _stream(stream)), "tq_encode_kv")


def tq_qjl_sketch(r, qjl_seed: int, bits, rnorm, stream=None):
    """bits [rows][d/32] int32 words, rnorm [rows] fp16 from residuals r [rows][d] fp32."""
    d = r.shape[-1]
    rows = r.numel() // d
    _check(_lib().tq_qjl_sketch(_ptr(r), rows, d, qjl_seed, _ptr(bits), _ptr(rnorm),
                                _stream(stream)), "tq_qjl_sketch")


def tq_attend_decode(cfg: Config, q, cache: PackedCache, n_ctx: int, out, ws,
                     scale: float = 0.0, splits: int = 0, stream=None):
    """out [B][Hq][d] fp32 = attention of q [B][Hq][d] over the first n_ctx tokens."""
    B, Hq, d = q.shape
    if d != cfg.d or not q.is_contiguous() or tuple(out.shape) != (B, Hq, d):
        raise TqError(TQ_ERR_ARG, "tq_attend_decode: q/out must be [B][Hq][d] contiguous")
    c = cache.c()
    _check(_lib().tq_attend_decode(ctypes.byref(cfg.c()), _ptr(q), _dtype_code(q), B, Hq,
                                   ctypes.byref(c), n_ctx, float(scale), splits, _ptr(out),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "tq_attend_decode")


def tq_attend_decode_noalloc(cfg: Config, q, cache: PackedCache, n_ctx: int, out,
                             scale: float = 0.0, splits: int = 0, stream=None):
    """tq_attend_decode without a workspace: the library's static per-GPU
    scratch buffer holds the split partials (calls must not overlap on one
    GPU)."""
    B, Hq, d = q.shape
    if d != cfg.d or not q.is_contiguous() or tuple(out.shape) != (B, Hq, d):
        raise TqError(TQ_ERR_ARG, "tq_attend_decode_noalloc: q/out must be [B][Hq][d] contiguous")
    c = cache.c()
    _check(_lib().tq_attend_decode_noalloc(ctypes.byref(cfg.c()), _ptr(q), _dtype_code(q), B, Hq,
                                           ctypes.byref(c), n_ctx, float(scale), splits, _ptr(out),
                                           _stream(stream)), "tq_attend_decode_noalloc")


def tq_dense_decode_bf16(q, k, v, out, ws, scale: float = 0.0, splits: int = 0, stream=None):
    """Dense bf16 decode baseline: q [B][Hq][d], k/v [B][Hkv][n][d] bf16, out fp32."""
    B, Hq, d = q.shape
    _, Hkv, n, _ = k.shape
    _check(_lib().tq_dense_decode_bf16(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, d, n,
                                       float(scale), splits, _ptr(out), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)),
           "tq_dense_decode_bf16")


def tq_append_attend_decode(cfg: Config, k_new, v_new, q, cache: PackedCache, n_ctx: int, out,
                            ws, scale: float = 0.0, splits: int = 0, stream=None):
    """Encode token n_ctx - 1 from k_new, v_new [B][Hkv][1][d], then attend
    like tq_attend_decode (one launch for 2/4-bit values without QJL)."""
    B, Hq, d = q.shape
    if d != cfg.d or not q.is_contiguous() or tuple(out.shape) != (B, Hq, d):
        raise TqError(TQ_ERR_ARG, "tq_append_attend_decode: q/out must be [B][Hq][d] contiguous")
    for t in (k_new, v_new):
        if tuple(t.shape) != (cache.B, cache.Hkv, 1, d) or not t.is_contiguous():
            raise TqError(TQ_ERR_ARG, "tq_append_attend_decode: k_new/v_new must be [B][Hkv][1][d]")
    if k_new.dtype != v_new.dtype:
        raise TqError(TQ_ERR_ARG, "tq_append_attend_decode: k_new and v_new dtypes differ")
    c = cache.c()
    _check(_lib().tq_append_attend_decode(
        ctypes.byref(cfg.c()), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(q),
        _dtype_code(q), B, Hq, ctypes.byref(c), n_ctx, float(scale), splits, _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)), "tq_append_attend_decode")


def tq_append_chunk_attend_decode(cfg: Config, k_new, v_new, q, cache: PackedCache, n_ctx: int,
                                  out, ws, scale: float = 0.0, splits: int = 0, stream=None):
    """Encode tokens n_ctx - n_new .. n_ctx - 1 from k_new, v_new
    [B][Hkv][n_new][d], then attend like tq_attend_decode (one launch on the
    matrix-core decode without QJL)."""
    B, Hq, d = q.shape
    if d != cfg.d or not q.is_contiguous() or tuple(out.shape) != (B, Hq, d):
        raise TqError(TQ_ERR_ARG,
                      "tq_append_chunk_attend_decode: q/out must be [B][Hq][d] contiguous")
    n_new = k_new.shape[2] if k_new.dim() == 4 else -1
    for t in (k_new, v_new):
        if tuple(t.shape) != (cache.B, cache.Hkv, n_new, d) or not t.is_contiguous():
            raise TqError(TQ_ERR_ARG, "tq_append_chunk_attend_decode: k_new/v_new must be "
                                      "contiguous [B][Hkv][n_new][d]")
    if k_new.dtype != v_new.dtype:
        raise TqError(TQ_ERR_ARG, "tq_append_chunk_attend_decode: k_new and v_new dtypes differ")
    c = cache.c()
    _check(_lib().tq_append_chunk_attend_decode(
        ctypes.byref(cfg.c()), _ptr(k_new), _ptr(v_new), _dtype_code(k_new), n_new, _ptr(q),
        _dtype_code(q), B, Hq, ctypes.byref(c), n_ctx, float(scale), splits, _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)), "tq_append_chunk_attend_decode")


def tq_attend_prefill(cfg: Config, q, cache: PackedCache, n_ctx: int, out, scale: float = 0.0,
                      stream=None):
    """Causal attention of the chunk q [B][Hq][n_q][d] (its tokens already at
    cache positions n_ctx - n_q .. n_ctx - 1) over the packed cache; out is
    [B][Hq][n_q][d] float32."""
    if q.dim() != 4 or q.shape[0] != cache.B or q.shape[3] != cfg.d or not q.is_contiguous():
        raise TqError(TQ_ERR_ARG, "tq_attend_prefill: q must be contiguous [B][Hq][n_q][d]")
    if tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise TqError(TQ_ERR_ARG, "tq_attend_prefill: out must be contiguous, shaped like q")
    c = cache.c()
    _check(_lib().tq_attend_prefill(ctypes.byref(cfg.c()), _ptr(q), _dtype_code(q), q.shape[0],
                                    q.shape[1], q.shape[2], ctypes.byref(c), n_ctx, scale,
                                    _ptr(out), _stream(stream)), "tq_attend_prefill")


def tq_read_probe(src, sink=None, stream=None):
    """Streaming read of every byte of the device tensor `src` (bandwidth
    probe); returns the sink tensor (one XOR word per wave)."""
    import torch
    nbytes = src.numel() * src.element_size()
    if not src.is_contiguous():
        raise TqError(TQ_ERR_ARG, "tq_read_probe: src must be contiguous")
    words = _check(_lib().tq_read_probe_sink_words(nbytes), "tq_read_probe_sink_words")
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=src.device)
    _check(_lib().tq_read_probe(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "tq_read_probe")
    return sink


def workspace(nbytes: int, device="cuda"):
    """A zeroed device byte buffer of at least nbytes (16-byte aligned by
    torch). Decode workspaces must be zero before their first use; the
    library leaves them that way after every call."""
    import torch
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# Group-affine variant (rotated keys, group 64, fp16 scale and bias)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class AffineConfig:
    d: int = 128
    bits_k: int = 4
    bits_v: int = 4
    group: int = 64
    seed: int = 0

    def c(self) -> tq_affine_config:
        return tq_affine_config(self.d, self.bits_k, self.bits_v, self.group, self.seed)


def tq_affine_cache_bytes(cfg: AffineConfig, B: int, Hkv: int, capacity: int):
    planes = (ctypes.c_int64 * 6)()
    total = _check(_lib().tq_affine_cache_bytes(ctypes.byref(cfg.c()), B, Hkv, capacity,
                                                ctypes.cast(planes, ctypes.c_void_p)),
                   "tq_affine_cache_bytes")
    return total, list(planes)


class AffineCache:
    """Device planes of an affine cache [B][Hkv][capacity]; see tq_affine_cache in tq.h."""

    def __init__(self, cfg: AffineConfig, B: int, Hkv: int, capacity: int, device="cuda"):
        import torch
        self.cfg, self.B, self.Hkv, self.capacity = cfg, B, Hkv, capacity
        _, p = tq_affine_cache_bytes(cfg, B, Hkv, capacity)
        shape = (B, Hkv, capacity)
        u8 = dict(dtype=torch.uint8, device=device)
        self.kc = torch.empty(shape + (cfg.d * cfg.bits_k // 8,), **u8)
        self.vc = torch.empty(shape + (cfg.d * cfg.bits_v // 8,), **u8)
        f16 = dict(dtype=torch.float16, device=device)
        ng = cfg.d // cfg.group
        self.ks, self.kb, self.vs, self.vb = (torch.empty(shape + (ng,), **f16) for _ in range(4))
        assert self.kc.numel() == p[0] and self.vc.numel() == p[1]
        assert all(t.numel() * 2 == p[2 + i]
                   for i, t in enumerate((self.ks, self.kb, self.vs, self.vb)))

    def c(self) -> tq_affine_cache:
        return tq_affine_cache(*(t.data_ptr() for t in
                                 (self.kc, self.vc, self.ks, self.kb, self.vs, self.vb)),
                               self.B, self.Hkv, self.capacity)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in
                   (self.kc, self.vc, self.ks, self.kb, self.vs, self.vb))


def tq_affine_encode_kv(cfg: AffineConfig, k, v, offset: int, cache: AffineCache, stream=None):
    """Encode k, v [B][Hkv][n_new][d] at token positions [offset, offset+n_new)."""
    if k.shape != v.shape or k.dtype != v.dtype:
        raise TqError(TQ_ERR_ARG, "tq_affine_encode_kv: k and v differ in shape or dtype")
    if k.dim() != 4 or k.shape[0] != cache.B or k.shape[1] != cache.Hkv or k.shape[3] != cfg.d:
        raise TqError(TQ_ERR_ARG, "tq_affine_encode_kv: k must be [B][Hkv][n_new][d]")
    if not (k.is_contiguous() and v.is_contiguous()):
        raise TqError(TQ_ERR_ARG, "tq_affine_encode_kv: k and v must be contiguous")
    c = cache.c()
    _check(_lib().tq_affine_encode_kv(ctypes.byref(cfg.c()), _ptr(k), _ptr(v), _dtype_code(k),
                                      offset, k.shape[2], ctypes.byref(c), _stream(stream)),
           "tq_affine_encode_kv")


def tq_affine_num_splits(cfg: AffineConfig, B, Hq, Hkv, n_ctx, splits=0):
    return _check(_lib().tq_affine_num_splits(ctypes.byref(cfg.c()), B, Hq, Hkv, n_ctx, splits),
                  "tq_affine_num_splits")


def tq_affine_workspace_bytes(cfg: AffineConfig, B, Hq, Hkv, n_ctx, splits=0):
    return _check(_lib().tq_affine_workspace_bytes(ctypes.byref(cfg.c()), B, Hq, Hkv, n_ctx,
                                                   splits), "tq_affine_workspace_bytes")


def tq_affine_attend_decode(cfg: AffineConfig, q, cache: AffineCache, n_ctx: int, out, ws,
                            scale: float = 0.0, splits: int = 0, stream=None):
    """out [B][Hq][d] fp32 = attention of q [B][Hq][d] over the first n_ctx affine tokens."""
    B, Hq, d = q.shape
    if d != cfg.d or not q.is_contiguous() or tuple(out.shape) != (B, Hq, d):
        raise TqError(TQ_ERR_ARG, "tq_affine_attend_decode: q/out must be [B][Hq][d] contiguous")
    c = cache.c()
    _check(_lib().tq_affine_attend_decode(ctypes.byref(cfg.c()), _ptr(q), _dtype_code(q), B, Hq,
                                          ctypes.byref(c), n_ctx, float(scale), splits,
                                          _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)), "tq_affine_attend_decode")
