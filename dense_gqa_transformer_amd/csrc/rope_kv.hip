// Per-head q/k RMSNorm + rotate-half RoPE + KV-cache write for a batch of
// prompt tokens.
//
// q/k RMSNorm over head_dim with one shared weight per projection, applied
// before RoPE (Qwen3 layout); RoPE pairs (i, i + r/2) of the first r dims
// rotated by p * theta^(-2i/r), r = head_dim or the partial width of the
// gated variant ("Failed Star (fs)", How it's built names RoPE; the
// rotate-half pairing and rotating 64 of 256 dims are what "ferrite", What it
// does, describes).  In the gated variant each head's q rows are followed by
// its gate rows in the projection output.  The cache
// keeps the normed, rotated K and the raw V ("Milestones", M4: cache K/V per layer).
#include "common.h"
#include "kernels.h"

namespace fsk {

// D/16 lanes per (token, head), 16 elements each: a rotated lane holds
// [8 sub, 8 sub + 8) and the matching RoPE partners [r/2 + 8 sub, ...), an
// unrotated one 16 consecutive dims from r on, so every access is a 16-byte
// vector and the rotation stays lane-local; 64/(D/16) heads per wave.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float* o) { load8(p, o); }
  static __device__ __forceinline__ void store(bf16* p, const float* v) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, (bf16)v[2 * i]);
      const uint32_t hi = __builtin_bit_cast(uint16_t, (bf16)v[2 * i + 1]);
      u[i] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(p) = u;
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* o) { load8(p, o); }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <typename TI, typename TQ, typename KV, int D>
__global__ __launch_bounds__(256) void rope_kv_kernel(const RopeKvParams p) {
  constexpr int LPH = D / 16;
  const int lane = threadIdx.x & 63, sub = lane % LPH;
  const int nh = p.nq + p.nkv;
  const long long item = ((long long)blockIdx.x * 256 + threadIdx.x) / LPH;
  const bool live = item < (long long)p.T * nh;
  const long long it = live ? item : 0;
  const int t = (int)(it / nh), hh = (int)(it % nh);
  const int b = t / p.S_per, pos = t % p.S_per;
  const int qmul = p.gated ? 2 : 1;                 // q rows interleaved with gate rows per head
  const int W = (p.nq * qmul + 2 * p.nkv) * D;
  const TI* row = reinterpret_cast<const TI*>(p.qkv) + (size_t)t * W;
  const bool is_q = hh < p.nq;
  const int j = hh - p.nq;
  const TI* src = is_q ? row + (size_t)hh * D * qmul : row + (size_t)p.nq * D * qmul + j * D;
  // the lane's 16 elements: rotated lanes (sub < rot/16) hold [8 sub, 8 sub + 8)
  // and their partners [rot/2 + 8 sub, ...); the others pass 16 consecutive
  // dims from rot on through unrotated
  const int R = p.rot, RH = R >> 1;
  const bool rotl = sub < (R >> 4);
  const int oA = rotl ? 8 * sub : R + 16 * (sub - (R >> 4));
  const int oB = rotl ? RH + 8 * sub : oA + 8;
  float x0[8], x1[8];
  Vec8<TI>::load(src + oA, x0);
  Vec8<TI>::load(src + oB, x1);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x0[e], x0[e], fmaf(x1[e], x1[e], ss));
  ss = group_sum<LPH>(ss);
  if (!live) return;
  const float inv = rsqrtf(__fadd_rn(ss / (float)D, p.eps));
  const float* g = is_q ? p.gq : p.gk;
  float g0[8], g1[8];
  load8(g + oA, g0);
  load8(g + oB, g1);
  float y0[8], y1[8];
  if (rotl) {
    float cs[8], sn[8];
    load8(p.cos_t + (size_t)pos * RH + 8 * sub, cs);
    load8(p.sin_t + (size_t)pos * RH + 8 * sub, sn);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // explicit fused multiply-adds: the QKV GEMM's fused epilogue computes the
      // same expressions and must round the same way
      const float a = x0[e] * inv * g0[e], c = x1[e] * inv * g1[e];
      y0[e] = fmaf(a, cs[e], -(c * sn[e]));
      y1[e] = fmaf(c, cs[e], a * sn[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) { y0[e] = x0[e] * inv * g0[e]; y1[e] = x1[e] * inv * g1[e]; }
  }
  if (is_q) {
#pragma unroll
    for (int e = 0; e < 8; ++e) { y0[e] *= p.qscale; y1[e] *= p.qscale; }
    TQ* q = reinterpret_cast<TQ*>(p.qout) + (size_t)t * p.nq * D + hh * D;
    Vec8<TQ>::store(q + oA, y0);
    Vec8<TQ>::store(q + oB, y1);
  } else {
    const int slot = p.slots[b];
    const size_t off = (size_t)slot * p.slot_stride + (size_t)j * p.head_stride + (size_t)pos * D;
    KV* k = reinterpret_cast<KV*>(p.kcache) + off;
    Vec8<KV>::store(k + oA, y0);
    Vec8<KV>::store(k + oB, y1);
    const TI* vs = row + (size_t)(p.nq * qmul + p.nkv) * D + j * D;
    float v0[8], v1[8];
    Vec8<TI>::load(vs + oA, v0);
    Vec8<TI>::load(vs + oB, v1);
    KV* v = reinterpret_cast<KV*>(p.vcache) + off;
    Vec8<KV>::store(v + oA, v0);
    Vec8<KV>::store(v + oB, v1);
  }
}

template <typename TI, typename TQ, typename KV>
static hipError_t launch_rope(const RopeKvParams& p, hipStream_t s) {
  const long long lanes = (long long)p.T * (p.nq + p.nkv) * (p.d / 16);
  const int blocks = (int)((lanes + 255) / 256);
  if (p.rot < 16 || p.rot > p.d || p.rot % 16 != 0) return hipErrorInvalidValue;
  if (p.d == 128)
    rope_kv_kernel<TI, TQ, KV, 128><<<blocks, 256, 0, s>>>(p);
  else if (p.d == 64)
    rope_kv_kernel<TI, TQ, KV, 64><<<blocks, 256, 0, s>>>(p);
  else if (p.d == 256)
    rope_kv_kernel<TI, TQ, KV, 256><<<blocks, 256, 0, s>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t rope_kv(const RopeKvParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  if (p.kv_dt == DT_BF16) {
    if (p.in_dt == DT_BF16 && p.q_dt == DT_BF16) return launch_rope<bf16, bf16, bf16>(p, s);
    if (p.in_dt == DT_F32 && p.q_dt == DT_F32) return launch_rope<float, float, bf16>(p, s);
    if (p.in_dt == DT_F32 && p.q_dt == DT_BF16) return launch_rope<float, bf16, bf16>(p, s);
  } else if (p.in_dt == DT_F32 && p.q_dt == DT_F32) {
    return launch_rope<float, float, float>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fsk
