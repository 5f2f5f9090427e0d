// Device code of libtq.so for gfx950 (CDNA4, wave64): helpers and kernel
// templates. Included by the kernel translation units only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace tq {
namespace dev {

constexpr float kLog2e = 1.4426950408889634f;

// Pointer into the constant address space: wave-uniform loads through it
// become scalar (SMEM) loads into SGPRs. Only for data the kernel never
// writes.
typedef const __attribute__((address_space(4))) float* const_f32_ptr;
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
__device__ __forceinline__ const_f32_ptr as_const(const float* p) {
  return (const_f32_ptr)(p);
}
__device__ __forceinline__ const_u32_ptr as_const(const uint32_t* p) {
  return (const_u32_ptr)(p);
}

// Two fp16 values in one dword (low half first) and their dot product with
// fp32 accumulation: v_dot2c_f32_f16.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                c, false);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return uint32_t(__builtin_bit_cast(uint16_t, _Float16(lo))) |
         (uint32_t(__builtin_bit_cast(uint16_t, _Float16(hi))) << 16);
}

// ---------------------------------------------------------------------------
// Element conversions (inputs are fp32, bf16 or fp16; bf16/fp16 arrive as
// raw 16-bit patterns).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return float(__builtin_bit_cast(_Float16, uint16_t(bits16)));
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, _Float16(x));
}

// Nearest-even rounding of a double to IEEE binary16, from the bit fields
// (one rounding step, so no double-rounding through fp32).
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
  const uint64_t b = uint64_t(__double_as_longlong(x));
  const uint16_t sign = uint16_t((b >> 48) & 0x8000u);
  const int e = int((b >> 52) & 0x7FF);
  const uint64_t m = b & ((uint64_t(1) << 52) - 1);
  if (e == 0x7FF) return sign | 0x7C00u | (m ? 0x200u : 0u);
  if (e == 0) return sign;
  const int E = e - 1023;
  if (E > 15) return sign | 0x7C00u;
  const uint64_t sig = m | (uint64_t(1) << 52);
  const int shift = (E >= -14) ? 42 : 28 - E;
  if (shift >= 54) return sign;
  uint64_t hs = sig >> shift;
  const uint64_t rem = sig & ((uint64_t(1) << shift) - 1);
  const uint64_t half = uint64_t(1) << (shift - 1);
  if (rem > half || (rem == half && (hs & 1))) ++hs;
  if (E >= -14) {
    int he = E + 15;
    if (hs == 2048) { hs = 1024; ++he; }
    if (he >= 31) return sign | 0x7C00u;
    return uint16_t(sign | (he << 10) | (hs & 0x3FF));
  }
  return uint16_t(sign | hs);
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) {
  return double(__builtin_bit_cast(_Float16, h));
}

// ---------------------------------------------------------------------------
// SplitMix64 as a counter-based generator: output i of the stream started at
// state `seed` (Steele, Lea, Flood, OOPSLA 2014). Rotation sign i is -1 when
// the top bit of output i is set.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Bit i of the result is 1 when sign(first + i) is negative, i < n <= 32.
__device__ __forceinline__ uint32_t sign_mask(uint64_t seed, int first, int n) {
  uint32_t m = 0;
  for (int i = 0; i < n; ++i)
    m |= uint32_t(splitmix64_at(seed, uint64_t(first + i)) >> 63) << i;
  return m;
}

// The same n bits (n <= 32, not crossing a 32-bit word) taken from a sign
// bitmap that the host filled from that stream (kernel argument, 8 words).
__device__ __forceinline__ uint32_t bitmap_bits(const uint32_t (&w)[8], int first, int n) {
  const int wi = first >> 5;
  uint32_t x = w[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) x = wi == k ? w[k] : x;
  x >>= (first & 31);
  return n == 32 ? x : (x & ((1u << n) - 1u));
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard transform of one row held by a group of 16 consecutive
// lanes, E consecutive elements per lane (row length 16*E). Element index
// l16*E + i; butterflies on index bit 0 first. Unnormalized (H_d x).
// ---------------------------------------------------------------------------

template <int E, typename T>
__device__ __forceinline__ void fwht16(T (&v)[E], int l16) {
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if (!(i & h)) {
        const T a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const T o = __shfl_xor(v[i], m, 16);
      v[i] = (l16 & m) ? (o - v[i]) : (v[i] + o);
    }
  }
}

__device__ __forceinline__ float group_max16(float x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 16));
  return x;
}

template <typename T>
__device__ __forceinline__ T group16_sum(T x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) x += __shfl_xor(x, m, 16);
  return x;
}

// Loads E consecutive elements of dtype `dt` (0 f32, 1 bf16, 2 f16) starting
// at element `idx` of `p` into floats. 16-byte aligned for E*size >= 16.
template <int E>
__device__ __forceinline__ void load_row_part(const void* p, int dt, int64_t idx,
                                              float (&f)[E]) {
  if (dt == 0) {
    const float4* s = reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
      const float4 q = s[k];
      f[4 * k + 0] = q.x; f[4 * k + 1] = q.y; f[4 * k + 2] = q.z; f[4 * k + 3] = q.w;
    }
  } else {
    const uint4* s = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + idx);
#pragma unroll
    for (int k = 0; k < E / 8; ++k) {
      const uint4 q = s[k];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = w[j] & 0xFFFFu, hi = w[j] >> 16;
        f[8 * k + 2 * j + 0] = dt == 1 ? bf16_to_f32(lo) : f16_to_f32(lo);
        f[8 * k + 2 * j + 1] = dt == 1 ? bf16_to_f32(hi) : f16_to_f32(hi);
      }
    }
  }
}

// The raw 16-byte words of E consecutive elements of dtype dt (0 f32, 1
// bf16, 2 f16) at element idx (E / 4 words for f32, E / 8 for 16-bit
// types), and their conversion to floats: the load and the conversion can
// then sit far apart.
template <int E>
__device__ __forceinline__ void load_row_raw(const void* p, int dt, int64_t idx,
                                             uint4 (&r)[E / 4]) {
  static_assert(E % 8 == 0, "whole 16-byte words");
  if (dt == 0) {
    const uint4* s = reinterpret_cast<const uint4*>(static_cast<const float*>(p) + idx);
#pragma unroll
    for (int k = 0; k < E / 4; ++k) r[k] = s[k];
  } else {
    const uint4* s = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + idx);
#pragma unroll
    for (int k = 0; k < E / 8; ++k) r[k] = s[k];
  }
}
template <int E>
__device__ __forceinline__ void convert_row_raw(const uint4 (&r)[E / 4], int dt, float (&f)[E]) {
  if (dt == 0) {
#pragma unroll
    for (int k = 0; k < E / 4; ++k) {
      f[4 * k] = __uint_as_float(r[k].x);
      f[4 * k + 1] = __uint_as_float(r[k].y);
      f[4 * k + 2] = __uint_as_float(r[k].z);
      f[4 * k + 3] = __uint_as_float(r[k].w);
    }
  } else {
#pragma unroll
    for (int k = 0; k < E / 8; ++k) {
      const uint32_t w[4] = {r[k].x, r[k].y, r[k].z, r[k].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = w[j] & 0xFFFFu, hi = w[j] >> 16;
        f[8 * k + 2 * j] = dt == 1 ? bf16_to_f32(lo) : f16_to_f32(lo);
        f[8 * k + 2 * j + 1] = dt == 1 ? bf16_to_f32(hi) : f16_to_f32(hi);
      }
    }
  }
}

// Field i (width BITS) of a little-endian bitstream held in dwords w[].
template <int BITS, int NW>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[NW], int i) {
  const int bit = i * BITS;
  const int wi = bit >> 5, sh = bit & 31;
  uint32_t x = w[wi] >> sh;
  if (sh + BITS > 32) x |= w[wi + 1] << (32 - sh);
  return BITS == 32 ? x : (x & ((1u << BITS) - 1u));
}

// The BITS-bit field that starts at bit `bit` of the words w (LSB-first),
// shifted left by P.
template <int BITS, int P, int NW>
__device__ __forceinline__ uint32_t bits_at(const uint32_t (&w)[NW], int bit) {
  const int wi = bit >> 5, sh = bit & 31;
  uint32_t x;
  if (sh + BITS > 32) {
    x = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], uint32_t(sh - P));
  } else if (sh >= P) {
    x = w[wi] >> (sh - P);
  } else {
    x = w[wi] << (P - sh);
  }
  return x & (((1u << BITS) - 1u) << P);
}

// Field i (width BITS) of the bitstream w[], already shifted left by P
// (result = field << P). Two VALU ops: one shift (or a funnel shift when the
// field straddles two dwords) and the mask. Needs P <= 32 - BITS... the
// straddling case needs the field to start at bit >= P of its dword.
template <int BITS, int P, int NW>
__device__ __forceinline__ uint32_t field_at(const uint32_t (&w)[NW], int i) {
  return bits_at<BITS, P>(w, i * BITS);
}

// Device-scope (agent) stores and loads of fp32 values: the stores write
// through this XCD's L2 and the loads do not hit a stale L2 line, so data a
// workgroup stores before an arrival count is read correctly by whichever
// workgroup, on whichever XCD, observes the count.
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev2(float* p, float x, float y) {
  const uint64_t v = uint64_t(__float_as_uint(x)) | (uint64_t(__float_as_uint(y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void load_dev2(const float* p, float* x, float* y) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  *x = __uint_as_float(uint32_t(v));
  *y = __uint_as_float(uint32_t(v >> 32));
}

// Raw buffer descriptor over [p, p + bytes): loads at byte offsets past the
// range return zero without touching memory (stride 0, 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), short(0), int(bytes),
                                           0x00020000);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// s[g] += dot2(q_g broadcast from lane L of every 16-lane row, c) for the
// G accumulators: v_dot2c_f32_f16 with a DPP row_newbcast source, so the
// query operand comes straight from a VGPR that only lane L of the row
// holds. The compiler checks no hazards inside inline assembly, so the
// block carries its own wait states:
//  * the leading s_nop 1 covers the DPP read of a VGPR written by a recent
//    VALU instruction (2 wait states);
//  * with TAIL, a trailing s_nop 4 covers a dot result read by a following
//    non-dot VALU instruction (CDNA3 asks for 3 wait states; only a dot that
//    takes it as its accumulator is interlocked). Chained calls accumulate
//    into s, so only the last call before s is read needs TAIL.
// EXEC must be full when this runs.
#define TQ_DOT2_DPP(D, Q, C, L) \
  "v_dot2c_f32_f16_dpp " D ", " Q ", " C " row_newbcast:" L " row_mask:0xf bank_mask:0xf\n\t"
template <int L, int G, bool TAIL = false>
__device__ __forceinline__ void dot2_bcast(float (&s)[G], const uint32_t (&q)[G], uint32_t c) {
  static_assert(G == 1 || G == 2 || G == 4, "G");
  if constexpr (G == 1) {
    if constexpr (TAIL)
      asm("s_nop 1\n\t" TQ_DOT2_DPP("%0", "%1", "%2", "%3") "s_nop 4"
          : "+v"(s[0]) : "v"(q[0]), "v"(c), "n"(L));
    else
      asm("s_nop 1\n\t" TQ_DOT2_DPP("%0", "%1", "%2", "%3")
          : "+v"(s[0]) : "v"(q[0]), "v"(c), "n"(L));
  } else if constexpr (G == 2) {
    if constexpr (TAIL)
      asm("s_nop 1\n\t" TQ_DOT2_DPP("%0", "%2", "%4", "%5") TQ_DOT2_DPP("%1", "%3", "%4", "%5")
          "s_nop 4"
          : "+v"(s[0]), "+v"(s[1]) : "v"(q[0]), "v"(q[1]), "v"(c), "n"(L));
    else
      asm("s_nop 1\n\t" TQ_DOT2_DPP("%0", "%2", "%4", "%5") TQ_DOT2_DPP("%1", "%3", "%4", "%5")
          : "+v"(s[0]), "+v"(s[1]) : "v"(q[0]), "v"(q[1]), "v"(c), "n"(L));
  } else {
    if constexpr (TAIL)
      asm("s_nop 1\n\t" TQ_DOT2_DPP("%0", "%4", "%8", "%9") TQ_DOT2_DPP("%1", "%5", "%8", "%9")
          TQ_DOT2_DPP("%2", "%6", "%8", "%9") TQ_DOT2_DPP("%3", "%7", "%8", "%9") "s_nop 4"
          : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3])
          : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(c), "n"(L));
    else
      asm("s_nop 1\n\t" TQ_DOT2_DPP("%0", "%4", "%8", "%9") TQ_DOT2_DPP("%1", "%5", "%8", "%9")
          TQ_DOT2_DPP("%2", "%6", "%8", "%9") TQ_DOT2_DPP("%3", "%7", "%8", "%9")
          : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3])
          : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(c), "n"(L));
  }
}
#undef TQ_DOT2_DPP

// Wave-wide max with DPP row operations (quad swaps, half-row and row
// mirrors, then row broadcasts); the result is taken from lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float x) {
  const int o = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL,
                                            ROW_MASK, 0xF, false);
  return fmaxf(x, __int_as_float(o));
}

__device__ __forceinline__ float dpp_wave_max(float v) {
  v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Stores `nbytes` low bytes of v at byte address p (alignment as stated).
__device__ __forceinline__ void store_bytes(uint8_t* p, uint64_t v, int nbytes) {
  switch (nbytes) {
    case 1: *p = uint8_t(v); break;
    case 2: *reinterpret_cast<uint16_t*>(p) = uint16_t(v); break;
    case 3: p[0] = uint8_t(v); p[1] = uint8_t(v >> 8); p[2] = uint8_t(v >> 16); break;
    case 4: *reinterpret_cast<uint32_t*>(p) = uint32_t(v); break;
    case 6: {
      uint16_t* q = reinterpret_cast<uint16_t*>(p);
      q[0] = uint16_t(v); q[1] = uint16_t(v >> 16); q[2] = uint16_t(v >> 32);
      break;
    }
    case 8: *reinterpret_cast<uint64_t*>(p) = v; break;
    default: break;
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Sums NV per-lane values over the 64 lanes of a wave, leaving the sums
// spread over the lanes ("transpose-reduce"). At lane-offset O the lane keeps
// the half of its CUR live values selected by (lane & O) and adds the
// partner's copy of that half; once one value is left, plain butterflies
// finish. reduce_index() gives the original index of each kept value.
template <int NV, int CUR, int O>
__device__ __forceinline__ void transpose_reduce_step(float (&v)[NV], int lane) {
  if constexpr (O >= 1) {
    if constexpr (CUR > 1) {
      constexpr int H = CUR / 2;
      const bool up = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[i + H];
        const float keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, O);
      }
      transpose_reduce_step<NV, H, O / 2>(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], O);
      transpose_reduce_step<NV, 1, O / 2>(v, lane);
    }
  }
}

template <int NV>
__device__ __forceinline__ void wave_transpose_reduce(float (&v)[NV], int lane) {
  transpose_reduce_step<NV, NV, 32>(v, lane);
}

// Values left per lane by wave_transpose_reduce<NV>.
template <int NV>
constexpr int reduce_kept() { return NV >= 64 ? NV / 64 : 1; }

// Original index of kept value i on `lane`, and whether this lane is the
// designated writer of it (several lanes hold copies when NV < 64).
template <int NV>
__device__ __forceinline__ int reduce_index(int lane, int i, bool* writer) {
  int cur = NV, idx = i;
  bool w = true;
  for (int o = 32; o >= 1; o >>= 1) {
    if (cur > 1) {
      const int half = cur >> 1;
      if (lane & o) idx += half;
      cur = half;
    } else if (lane & o) {
      w = false;
    }
  }
  *writer = w;
  return idx;
}

}  // namespace dev
}  // namespace tq
