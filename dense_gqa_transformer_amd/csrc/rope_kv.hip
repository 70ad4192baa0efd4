// Per-head q/k RMSNorm + rotate-half RoPE + KV-cache write for a batch of
// prompt tokens.  One wave per (token, head); lane l holds the RoPE pair
// (l, l + d/2), so the rotation is lane-local and the norm is one wave sum.
//
// q/k RMSNorm over head_dim with one shared weight per projection, applied
// before RoPE (Qwen3 layout); RoPE pairs (i, i + d/2) rotated by
// p * theta^(-2i/d) ("Failed Star (fs)", How it's built names RoPE; the
// rotate-half pairing is the one "ferrite", What it does, names).  The cache
// keeps the normed, rotated K and the raw V ("Milestones", M4: cache K/V per layer).
#include "common.h"
#include "kernels.h"

namespace fsk {

template <typename TI, typename TQ, typename KV>
__global__ __launch_bounds__(256) void rope_kv_kernel(const RopeKvParams p) {
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nh = p.nq + p.nkv;
  const long long item = (long long)blockIdx.x * 4 + wid;
  if (item >= (long long)p.T * nh) return;
  const int t = (int)(item / nh), hh = (int)(item % nh);
  const int d = p.d, half = d >> 1;
  const int b = t / p.S_per, pos = t % p.S_per;
  const int slot = p.slots[b];
  const int W = (p.nq + 2 * p.nkv) * d;
  const TI* row = reinterpret_cast<const TI*>(p.qkv) + (size_t)t * W;
  const bool on = lane < half;
  const bool is_q = hh < p.nq;
  const int j = hh - p.nq;
  const TI* src = is_q ? row + hh * d : row + p.nq * d + j * d;
  float x0 = on ? to_f32(src[lane]) : 0.f;
  float x1 = on ? to_f32(src[lane + half]) : 0.f;
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float inv = rsqrtf(ss / (float)d + p.eps);
  const float* g = is_q ? p.gq : p.gk;
  if (on) {
    x0 = x0 * inv * g[lane];
    x1 = x1 * inv * g[lane + half];
    const float c = p.cos_t[(size_t)pos * half + lane];
    const float s = p.sin_t[(size_t)pos * half + lane];
    const float y0 = x0 * c - x1 * s;
    const float y1 = x1 * c + x0 * s;
    if (is_q) {
      TQ* q = reinterpret_cast<TQ*>(p.qout) + (size_t)t * p.nq * d + hh * d;
      q[lane] = from_f32<TQ>(y0);
      q[lane + half] = from_f32<TQ>(y1);
    } else {
      const size_t off = (size_t)slot * p.slot_stride + (size_t)j * p.head_stride + (size_t)pos * d;
      KV* k = reinterpret_cast<KV*>(p.kcache) + off;
      k[lane] = from_f32<KV>(y0);
      k[lane + half] = from_f32<KV>(y1);
      const TI* vs = row + (p.nq + p.nkv) * d + j * d;
      KV* v = reinterpret_cast<KV*>(p.vcache) + off;
      v[lane] = from_f32<KV>(to_f32(vs[lane]));
      v[lane + half] = from_f32<KV>(to_f32(vs[lane + half]));
    }
  }
}

hipError_t rope_kv(const RopeKvParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  if (p.d > 128 || (p.d & 1)) return hipErrorInvalidValue;
  const long long items = (long long)p.T * (p.nq + p.nkv);
  const int blocks = (int)((items + 3) / 4);
  if (p.kv_dt == DT_BF16) {
    if (p.in_dt == DT_BF16 && p.q_dt == DT_BF16)
      rope_kv_kernel<bf16, bf16, bf16><<<blocks, 256, 0, s>>>(p);
    else if (p.in_dt == DT_F32 && p.q_dt == DT_F32)
      rope_kv_kernel<float, float, bf16><<<blocks, 256, 0, s>>>(p);
    else
      return hipErrorInvalidValue;
  } else {
    if (p.in_dt == DT_F32 && p.q_dt == DT_F32)
      rope_kv_kernel<float, float, float><<<blocks, 256, 0, s>>>(p);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fsk
