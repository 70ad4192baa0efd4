// Shared device helpers for the gfx950 kernels (wave64, CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define WAVE 64

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Cross-lane reductions on DPP row operations (no LDS round trip): within an
// aligned row of 16 lanes, exchange with lane ^ 1 and lane ^ 2 (quad
// permutes), then with the mirrored lane of the half row and of the row, so
// every lane of the row ends with the row's total; whole-wave results then
// combine row pairs and wave halves with the permlane swaps below.  Every lane
// of the wave (or row) must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);     // quad_perm(1, 0, 3, 2)
  v += dpp_f<0x4E>(v);     // quad_perm(2, 3, 0, 1)
  v += dpp_f<0x141>(v);    // row_half_mirror
  v += dpp_f<0x140>(v);    // row_mirror
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}
// Across rows, v_permlane16_swap / v_permlane32_swap (gfx950) with both
// operands v return, in every lane, the two values of its xor-16 (xor-32) pair:
// first the lower lane's, then the upper lane's.
struct LanePair { float lo, hi; };
__device__ __forceinline__ LanePair pair16(float v) {
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(q[0]), __uint_as_float(q[1])};
}
__device__ __forceinline__ LanePair pair32(float v) {
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return {__uint_as_float(q[0]), __uint_as_float(q[1])};
}
// the value held by lane ^ 16 / lane ^ 32
__device__ __forceinline__ float xor16_f(float v) {
  const LanePair p = pair16(v);
  return (__lane_id() & 16) ? p.lo : p.hi;
}
__device__ __forceinline__ float xor32_f(float v) {
  const LanePair p = pair32(v);
  return (__lane_id() & 32) ? p.lo : p.hi;
}
__device__ __forceinline__ float pair32_sum(float v) {
  const LanePair p = pair32(v);
  return p.lo + p.hi;
}
__device__ __forceinline__ float pair32_max(float v) {
  const LanePair p = pair32(v);
  return fmaxf(p.lo, p.hi);
}

// Sum over the 64 lanes of a wave (every lane receives the total).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  const LanePair r = pair16(v);
  return pair32_sum(r.lo + r.hi);
}

// Sum over aligned groups of `W` lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W == 16) {
    return row16_sum(v);
  } else if constexpr (W == 64) {
    return wave_sum(v);
  } else {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
  }
}

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  const LanePair r = pair16(v);
  return pair32_max(fmaxf(r.lo, r.hi));
}

// Loads 8 consecutive elements as fp32 (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ void load8(const bf16* p, float* out) {
  u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(u[i] << 16);
    out[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// The four signed 8-bit codes packed in a 32-bit word, as fp32 (exact).
__device__ __forceinline__ void codes4(uint32_t w, float* out) {
#pragma unroll
  for (int b = 0; b < 4; ++b) out[b] = (float)(int)(int8_t)(uint8_t)(w >> (8 * b));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// (value, index) ordering for greedy selection: larger finite value wins,
// the lower index wins an exact tie; non-finite values never win.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  if (bi < 0) return i >= 0;
  if (i < 0) return false;
  return v > bv || (v == bv && i < bi);
}

// ---------------------------------------------------------------- fp8 (e4m3)
// 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities, largest 448:
// the operand format of the gfx950 fp8 matrix instructions.
// Nearest e4m3 code of x (ties to an even mantissa, magnitudes past 448
// saturate, a zero result is code 0 whatever the sign); x finite.
__device__ __forceinline__ uint32_t f8_encode(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), 448.f);
  if (a < 0.015625f) {                               // below 2^-6: steps of 2^-9 (8 -> the smallest normal)
    const uint32_t m = (uint32_t)(int)rintf(a * 512.f);
    return m ? (sign | m) : 0u;
  }
  const uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xFF) - 127;            // -6 .. 8
  uint32_t keep = (u >> 20) & 7u;
  const uint32_t rest = u & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) { keep = 0u; ++e; }
  return sign | ((uint32_t)(e + 7) << 3) | keep;
}
// value of an e4m3 code (exact in fp32)
__device__ __forceinline__ float f8_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}
// Row scale of the fp8 rule: the smallest power of two >= fl(amax / 448), 0 for amax 0.
__device__ __forceinline__ float f8_row_scale(float amax) {
  if (!(amax > 0.f)) return 0.f;
  const float t = amax / 448.f;
  const uint32_t u = __float_as_uint(t);
  const uint32_t ex = (u >> 23) & 0xFF, man = u & 0x7FFFFF;
  if (ex != 0) return man == 0 ? t : __uint_as_float((ex + 1u) << 23);
  return man == 1u ? ldexpf(1.f, -149) : ldexpf(1.f, 32 - __builtin_clz(man - 1u) - 149);   // t subnormal
}

// Causal prefill attention grids: workgroup L of a 1-D grid of nqt * ny * nb
// takes query tile qt of head group y of sequence b, in order of decreasing
// work across all heads and sequences (query tile qt reads qt + 1 key tiles),
// so that the longest tiles start first and the short ones fill the tail.
__device__ __forceinline__ void longest_first(int L, int nqt, int ny, int nb, int& qt, int& y, int& b) {
  const int per = ny * nb;
  const int g = L / per, r = L - g * per;
  qt = nqt - 1 - g;
  y = r % ny;
  b = r / ny;
}
