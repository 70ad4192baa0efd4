// Small bandwidth-bound kernels: embedding gather, RMSNorm, dtype widening,
// gate/up packing and row argmax.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace fsk {

__device__ __forceinline__ float block_sum256(float v, float* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  v = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return v;
}

// ------------------------------------------------------------------ embedding
// Token embedding gather ("Coming back to Failed Star", Second sitting:
// ids[S] -> embedding[S,H]); the residual stream is kept in fp32.
template <typename W>
__global__ __launch_bounds__(256) void embed_kernel(const W* __restrict__ E, const int32_t* __restrict__ tok,
                                                    int H, int V, float* __restrict__ x) {
  const int t = blockIdx.x;
  int id = tok[t];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  const W* row = E + (size_t)id * H;
  float* dst = x + (size_t)t * H;
  for (int k = threadIdx.x * 8; k < H; k += 256 * 8) {
    float v[8];
    load8(row + k, v);
    *reinterpret_cast<float4*>(dst + k) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(dst + k + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// int8 rows: code * the row's scale, rounded to fp32 (the residual stream)
__global__ __launch_bounds__(256) void embed_i8_kernel(const int8_t* __restrict__ E,
                                                       const float* __restrict__ escale,
                                                       const int32_t* __restrict__ tok, int H, int V,
                                                       float* __restrict__ x) {
  const int t = blockIdx.x;
  int id = tok[t];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  const int8_t* row = E + (size_t)id * H;
  const float sc = escale[id];
  float* dst = x + (size_t)t * H;
  for (int k = threadIdx.x * 8; k < H; k += 256 * 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + k);
    float v[8];
    codes4(w.x, v);
    codes4(w.y, v + 4);
    *reinterpret_cast<float4*>(dst + k) = make_float4(v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc);
    *reinterpret_cast<float4*>(dst + k + 4) = make_float4(v[4] * sc, v[5] * sc, v[6] * sc, v[7] * sc);
  }
}

hipError_t embed(const void* E, int dt, const int32_t* tok, int T, int H, int V, float* x, hipStream_t s,
                 const float* escale) {
  if (T <= 0) return hipSuccess;
  if (dt == DT_I8) {
    if (escale == nullptr || H % 8 != 0) return hipErrorInvalidValue;
    embed_i8_kernel<<<T, 256, 0, s>>>((const int8_t*)E, escale, tok, H, V, x);
  } else if (dt == DT_BF16) {
    embed_kernel<bf16><<<T, 256, 0, s>>>((const bf16*)E, tok, H, V, x);
  } else {
    embed_kernel<float><<<T, 256, 0, s>>>((const float*)E, tok, H, V, x);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ int8 rows
// Per-row symmetric quantization, one wave per row: the row's largest
// magnitude (wave max), scale = amax / 127 and code = rint(x / scale), both
// quotients correctly rounded fp32 divisions.  Rows are re-read for the
// codes (they are a few KB and still in cache).
template <typename W>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const W* __restrict__ src, int rows, int cols,
                                                            int8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const W* row = src + (size_t)r * cols;
  float amax = 0.f;
  for (int k = lane * 8; k < cols; k += 64 * 8) {
    float v[8];
    load8(row + k, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
  amax = wave_max(amax);
  const float sc = amax / 127.0f;
  if (lane == 0) scales[r] = sc;
  int8_t* out = codes + (size_t)r * cols;
  for (int k = lane * 8; k < cols; k += 64 * 8) {
    float v[8];
    load8(row + k, v);
    uint32_t w[2] = {0u, 0u};
    if (sc > 0.f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float q = fminf(fmaxf(rintf(v[e] / sc), -127.f), 127.f);
        w[e >> 2] |= (uint32_t)(uint8_t)(int8_t)(int)q << (8 * (e & 3));
      }
    }
    *reinterpret_cast<uint2*>(out + k) = make_uint2(w[0], w[1]);
  }
}

hipError_t quantize_rows(const void* src, int dt, int rows, int cols, int8_t* codes, float* scales,
                         hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (cols <= 0 || cols % 8 != 0) return hipErrorInvalidValue;
  const int blocks = (rows + 3) / 4;
  if (dt == DT_BF16)
    quantize_rows_kernel<bf16><<<blocks, 256, 0, s>>>((const bf16*)src, rows, cols, codes, scales);
  else if (dt == DT_F32)
    quantize_rows_kernel<float><<<blocks, 256, 0, s>>>((const float*)src, rows, cols, codes, scales);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Codes as bf16 operands of the MFMA GEMM (integers up to 127 are exact).
__global__ __launch_bounds__(256) void codes_to_bf16_kernel(const int8_t* __restrict__ codes, size_t n16,
                                                            bf16* __restrict__ dst) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(codes + i * 16);
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) codes4(w[j], v + 4 * j);
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a[e] = (bf16)v[e]; b[e] = (bf16)v[8 + e]; }
    *reinterpret_cast<bf16x8*>(dst + i * 16) = a;
    *reinterpret_cast<bf16x8*>(dst + i * 16 + 8) = b;
  }
}

hipError_t codes_to_bf16(const int8_t* codes, size_t n, void* dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (n % 16 != 0) return hipErrorInvalidValue;
  const size_t n16 = n / 16;
  const size_t blocks = std::min<size_t>((n16 + 255) / 256, 4096);
  codes_to_bf16_kernel<<<(unsigned)blocks, 256, 0, s>>>(codes, n16, (bf16*)dst);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// x / sqrt(mean(x^2) + eps) * g over one row ("Failed Star (fs)", How it's built).
// With `lo` set (bf16 output only) the value is also split: out = bf16(y),
// lo = bf16(y - out), so that out + lo carries y to about 16 significant bits.
// One wave per row: lane l holds the 16-byte chunks l, l + 64, ... of the row
// in registers (one read of x), the mean square is one wave sum, and the
// outputs leave as 8- or 16-byte stores.
template <typename O>
__device__ __forceinline__ void norm_store(const f32x4& v, float inv, const float* g, int c, O* o, O* lo) {
  const f32x4 gg = *reinterpret_cast<const f32x4*>(g + 4 * c);
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = v[e] * inv * gg[e];
  if constexpr (sizeof(O) == 2) {
    bf16x4 hi, rem;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = (bf16)y[e];
      rem[e] = (bf16)(y[e] - (float)hi[e]);
    }
    *reinterpret_cast<bf16x4*>(o + 4 * c) = hi;
    if (lo != nullptr) *reinterpret_cast<bf16x4*>(lo + 4 * c) = rem;
  } else {
    *reinterpret_cast<f32x4*>(o + 4 * c) = f32x4{y[0], y[1], y[2], y[3]};
  }
}

template <typename O, int MAXJ>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int T, int H, int ldx,
                                                      const float* __restrict__ g, float eps,
                                                      O* __restrict__ out, O* __restrict__ lo, int ldo) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= T) return;
  const float* row = x + (size_t)r * ldx;
  const int nc = H >> 2;
  f32x4 v[MAXJ];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int c = lane + 64 * j;
    v[j] = (c < nc) ? *reinterpret_cast<const f32x4*>(row + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(v[j][e], v[j][e], ss);
  }
  const float inv = rsqrtf(wave_sum(ss) / (float)H + eps);
  O* o = out + (size_t)r * ldo;
  O* ol = (lo != nullptr) ? lo + (size_t)r * ldo : nullptr;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int c = lane + 64 * j;
    if (c >= nc) break;
    norm_store<O>(v[j], inv, g, c, o, ol);
  }
}

// With split-K partials to add: one workgroup per row, thread t holding the
// 16-byte chunks t, t + 256, ...; each chunk's np partial loads go out
// together, the partials are added in order 0..np-1 (so the result does not
// depend on launch timing) and the row is written back before it is
// normalised (out == nullptr: the additions only).
template <typename O>
__global__ __launch_bounds__(256) void rmsnorm_add_kernel(float* __restrict__ x, int T, int H, int ldx,
                                                          const float* __restrict__ g, float eps,
                                                          O* __restrict__ out, O* __restrict__ lo, int ldo,
                                                          const float* __restrict__ parts, int np) {
  constexpr int MAXC = 4;                          // H <= 4096
  __shared__ float red[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  float* row = x + (size_t)r * ldx;
  const int nc = H >> 2;
  const size_t pst = (size_t)T * H;
  const float* prow = parts + (size_t)r * H;
  f32x4 v[MAXC];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int c = tid + 256 * j;
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c < nc) {
      f32x4 pv[RMSNORM_MAX_PARTS];
#pragma unroll
      for (int q = 0; q < RMSNORM_MAX_PARTS; ++q)
        if (q < np) pv[q] = *reinterpret_cast<const f32x4*>(prow + q * pst + 4 * c);
      f32x4 a = *reinterpret_cast<const f32x4*>(row + 4 * c);
#pragma unroll
      for (int q = 0; q < RMSNORM_MAX_PARTS; ++q)
        if (q < np) a += pv[q];
      *reinterpret_cast<f32x4*>(row + 4 * c) = a;
      v[j] = a;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(v[j][e], v[j][e], ss);
  }
  if (out == nullptr) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float inv = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  O* o = out + (size_t)r * ldo;
  O* ol = (lo != nullptr) ? lo + (size_t)r * ldo : nullptr;
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int c = tid + 256 * j;
    if (c < nc) norm_store<O>(v[j], inv, g, c, o, ol);
  }
}

hipError_t rmsnorm(const float* x, int T, int H, int ldx, const float* g, float eps, void* out,
                   int out_dt, int ldo, hipStream_t s, void* lo) {
  if (T <= 0) return hipSuccess;
  if (out == nullptr || H % 4 != 0 || H > 4096 || ldx % 4 != 0 || ldo % 4 != 0) return hipErrorInvalidValue;
  const int blocks = (T + 3) / 4;
  if (out_dt == DT_BF16)
    rmsnorm_kernel<bf16, 16><<<blocks, 256, 0, s>>>(x, T, H, ldx, g, eps, (bf16*)out, (bf16*)lo, ldo);
  else if (lo == nullptr)
    rmsnorm_kernel<float, 16><<<blocks, 256, 0, s>>>(x, T, H, ldx, g, eps, (float*)out, nullptr, ldo);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t rmsnorm_add(float* x, const float* parts, int np, int T, int H, int ldx, const float* g, float eps,
                       void* out, int out_dt, int ldo, hipStream_t s, void* lo) {
  if (T <= 0) return hipSuccess;
  if (np <= 0 || np > RMSNORM_MAX_PARTS || parts == nullptr) return hipErrorInvalidValue;
  if (H % 4 != 0 || H > 4096 || ldx % 4 != 0 || ldo % 4 != 0) return hipErrorInvalidValue;
  if (out_dt == DT_BF16)
    rmsnorm_add_kernel<bf16><<<T, 256, 0, s>>>(x, T, H, ldx, g, eps, (bf16*)out, (bf16*)lo, ldo, parts, np);
  else if (lo == nullptr)
    rmsnorm_add_kernel<float><<<T, 256, 0, s>>>(x, T, H, ldx, g, eps, (float*)out, nullptr, ldo, parts, np);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ widening
template <typename W>
__global__ void convert_kernel(const W* __restrict__ src, float* __restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = to_f32(src[i]);
}

hipError_t convert_f32(const void* src, int dt, float* dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256);
  if (dt == DT_BF16)
    convert_kernel<bf16><<<blocks, 256, 0, s>>>((const bf16*)src, dst, n);
  else
    convert_kernel<float><<<blocks, 256, 0, s>>>((const float*)src, dst, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ timing gate
// Waits a bounded time on the device wall clock (100 MHz on this target).
__global__ void spin_wait_kernel(long long ticks) {
  const long long t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

hipError_t spin_wait(int us, hipStream_t s) {
  spin_wait_kernel<<<1, 64, 0, s>>>((long long)us * 100);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gate/up packing
template <typename W>
__global__ void pack_gate_up_kernel(const W* __restrict__ gate, const W* __restrict__ up, int H,
                                    W* __restrict__ dst) {
  const int r = blockIdx.x;                // packed row in [0, 2I)
  const int blk = r >> 6, within = r & 63;
  const W* src = (within < 32 ? gate : up) + (size_t)(blk * 32 + (within & 31)) * H;
  W* d = dst + (size_t)r * H;
  for (int k = threadIdx.x; k < H; k += blockDim.x) d[k] = src[k];
}

hipError_t pack_gate_up(const void* gate, const void* up, int dt, int I, int H, void* dst, hipStream_t s) {
  if (dt == DT_BF16)
    pack_gate_up_kernel<bf16><<<2 * I, 256, 0, s>>>((const bf16*)gate, (const bf16*)up, H, (bf16*)dst);
  else
    pack_gate_up_kernel<float><<<2 * I, 256, 0, s>>>((const float*)gate, (const float*)up, H, (float*)dst);
  return hipGetLastError();
}

// ------------------------------------------------------------------ argmax
// Greedy selection ("Coming back to Failed Star", section Next): the largest
// finite logit, lowest ID on an exact tie, -1 when no logit is finite.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ logits, int V, int ldl,
                                                      int32_t* __restrict__ out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const float* row = logits + (size_t)blockIdx.x * ldl;
  float bv = 0.f;
  int bi = -1;
  for (int i = threadIdx.x; i < V; i += 1024) {
    const float v = row[i];
    if (__builtin_isfinite(v) && better(v, i, bv, bi)) { bv = v; bi = i; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) { sv[wid] = bv; si[wid] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    out[blockIdx.x] = bi;
  }
}

hipError_t argmax_rows(const float* logits, int B, int V, int ldl, int32_t* out, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  argmax_kernel<<<B, 1024, 0, s>>>(logits, V, ldl, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- attention output gate
// a[t, h*d + e] *= sigmoid(qkv[t, 2h*d + d + e]): the gated-attention variant's
// per-head output gate, read from the gate rows the q projection interleaves
// with each head's query rows ("ferrite", What it does).
template <typename TA, typename TG>
__global__ __launch_bounds__(256) void attn_gate_kernel(TA* __restrict__ a, const TG* __restrict__ qkv, int T,
                                                        int nq, int d, int ldq) {
  const long long n = (long long)T * nq * d;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const int t = (int)(i / ((long long)nq * d));
    const int r = (int)(i % ((long long)nq * d));
    const int h = r / d, e = r % d;
    const float g = to_f32(qkv[(size_t)t * ldq + (size_t)(2 * h + 1) * d + e]);
    a[i] = from_f32<TA>(to_f32(a[i]) / (1.f + __expf(-g)));
  }
}

hipError_t attn_gate(void* a, int a_dt, const void* qkv, int qkv_dt, int T, int nq, int d, int ldq,
                     hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const long long n = (long long)T * nq * d;
  const int blocks = (int)std::min<long long>((n + 255) / 256, 4096);
  if (a_dt == DT_BF16 && qkv_dt == DT_BF16)
    attn_gate_kernel<bf16, bf16><<<blocks, 256, 0, s>>>((bf16*)a, (const bf16*)qkv, T, nq, d, ldq);
  else if (a_dt == DT_BF16 && qkv_dt == DT_F32)
    attn_gate_kernel<bf16, float><<<blocks, 256, 0, s>>>((bf16*)a, (const float*)qkv, T, nq, d, ldq);
  else if (a_dt == DT_F32 && qkv_dt == DT_F32)
    attn_gate_kernel<float, float><<<blocks, 256, 0, s>>>((float*)a, (const float*)qkv, T, nq, d, ldq);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fsk
