// Bandwidth-bound GEMV for the decode path and other calls with few rows.
//
// y[m, n] = sum_k W[n, k] * a[m, k], with W stored [out, in] ("Coming back to
// Failed Star", First sitting, item 3).  Each workgroup stages its activation
// rows in LDS (optionally RMS-normalised, fused prologue), then each wave
// streams RPW weight rows with 16-byte loads, lane l covering the 8-element
// chunks l, l+64, l+128, ...  The cross-lane sum is a wave64 shuffle tree.
// Epilogues: plain store, residual add, SwiGLU on paired gate/up rows, and
// lm_head logits with a block argmax reduced by the last workgroup.
#include "common.h"
#include "kernels.h"

namespace fsk {

static constexpr int GEMV_THREADS = 256;
static constexpr int GEMV_WAVES = 4;

template <typename W> struct Raw;
template <> struct Raw<bf16> { u32x4 v; };
template <> struct Raw<float> { f32x4 a, b; };

__device__ __forceinline__ void raw_load(const bf16* p, Raw<bf16>& r) {
  r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void raw_load(const float* p, Raw<float>& r) {
  r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
}
__device__ __forceinline__ void raw_zero(Raw<bf16>& r) { r.v = u32x4{0, 0, 0, 0}; }
__device__ __forceinline__ void raw_zero(Raw<float>& r) { r.a = f32x4{0, 0, 0, 0}; r.b = r.a; }
__device__ __forceinline__ void raw_f32(const Raw<bf16>& r, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(r.v[i] << 16);
    o[2 * i + 1] = __uint_as_float(r.v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void raw_f32(const Raw<float>& r, float* o) {
  o[0] = r.a[0]; o[1] = r.a[1]; o[2] = r.a[2]; o[3] = r.a[3];
  o[4] = r.b[0]; o[5] = r.b[1]; o[6] = r.b[2]; o[7] = r.b[3];
}

// Weight row for the i-th row slot of a wave.  SWIGLU: "rows" walk features,
// even slots read the gate row and odd slots the up row of the packed matrix.
template <int EPI>
__device__ __forceinline__ int weight_row(int slot_row, int& feature) {
  if (EPI == EPI_SWIGLU) {
    feature = slot_row >> 1;
    return ((feature >> 5) << 6) + (feature & 31) + ((slot_row & 1) << 5);
  }
  feature = slot_row;
  return slot_row;
}

template <typename W, int EPI, int MB, int CPL, int RPW>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_kernel(const GemvParams p) {
  extern __shared__ float lds[];          // [MB][K] activations, then 2*16 reduce scratch
  const int K = p.K;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int m0 = blockIdx.y * MB;
  const int mcount = min(MB, p.M - m0);
  float* red = lds + MB * K;

  // ---- prologue: stage (and optionally RMS-normalise) the activation rows
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const bool live = m < mcount;
    const float* arow = p.a + (size_t)(m0 + (live ? m : 0)) * p.lda;
    float ss = 0.f;
    for (int k = tid; k < K; k += GEMV_THREADS) {
      const float v = live ? arow[k] : 0.f;
      lds[m * K + k] = v;
      ss += v * v;
    }
    if (p.gamma != nullptr) {
      ss = wave_sum(ss);
      if (lane == 0) red[m * 4 + wid] = ss;
    }
  }
  if (p.gamma != nullptr) {
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float ss = red[m * 4] + red[m * 4 + 1] + red[m * 4 + 2] + red[m * 4 + 3];
      const float inv = rsqrtf(ss / (float)K + p.eps);
      for (int k = tid; k < K; k += GEMV_THREADS) lds[m * K + k] *= inv * p.gamma[k];
    }
  }
  __syncthreads();

  const W* __restrict__ w = reinterpret_cast<const W*>(p.w);
  const int nchunk = K >> 3;
  const int slots_total = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;   // weight rows to cover
  const int rows_per_block = GEMV_WAVES * RPW * p.groups;

  float best_v[MB];
  int best_i[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) { best_v[m] = 0.f; best_i[m] = -1; }

  for (int g = 0; g < p.groups; ++g) {
    const int rbase = blockIdx.x * rows_per_block + (g * GEMV_WAVES + wid) * RPW;
    if (rbase >= slots_total) break;
    // ---- issue every weight load of this row group first
    Raw<W> raw[CPL][RPW];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        int f;
        const int r = weight_row<EPI>(rbase + i, f);
        if (c < nchunk && rbase + i < slots_total)
          raw_load(w + (size_t)r * K + c * 8, raw[j][i]);
        else
          raw_zero(raw[j][i]);
      }
    }
    // ---- multiply-accumulate against the staged activations
    float acc[RPW][MB];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[i][m] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunk) {
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const float4 a0 = *reinterpret_cast<const float4*>(lds + m * K + c * 8);
          const float4 a1 = *reinterpret_cast<const float4*>(lds + m * K + c * 8 + 4);
#pragma unroll
          for (int i = 0; i < RPW; ++i) {
            float wv[8];
            raw_f32(raw[j][i], wv);
            float s = acc[i][m];
            s = fmaf(wv[0], a0.x, s); s = fmaf(wv[1], a0.y, s);
            s = fmaf(wv[2], a0.z, s); s = fmaf(wv[3], a0.w, s);
            s = fmaf(wv[4], a1.x, s); s = fmaf(wv[5], a1.y, s);
            s = fmaf(wv[6], a1.z, s); s = fmaf(wv[7], a1.w, s);
            acc[i][m] = s;
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[i][m] = wave_sum(acc[i][m]);

    // ---- epilogue (lane 0 of each wave holds the sums)
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int sr = rbase + i;
        if (sr >= slots_total) continue;
        int f;
        weight_row<EPI>(sr, f);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m >= mcount) continue;
          const size_t o = (size_t)(m0 + m) * p.ldo + f;
          if (EPI == EPI_STORE) {
            p.out[o] = acc[i][m];
          } else if (EPI == EPI_RESID) {
            p.out[o] += acc[i][m];
          } else if (EPI == EPI_SWIGLU) {
            // slot rows come in (gate, up) pairs: i even = gate, i + 1 = up
            if ((i & 1) == 0) p.out[o] = silu(acc[i][m]) * acc[(i + 1) % RPW][m];
          } else {  // EPI_LOGITS
            const float v = acc[i][m];
            if (p.logits) p.logits[o] = v;
            if (__builtin_isfinite(v) && better(v, f, best_v[m], best_i[m])) { best_v[m] = v; best_i[m] = f; }
          }
        }
      }
    }
  }

  if (EPI == EPI_LOGITS) {
    // block-level best per row, then the last block reduces all blocks
    __shared__ float bvs[GEMV_WAVES][MB];
    __shared__ int bis[GEMV_WAVES][MB];
    __shared__ bool last;
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m) { bvs[wid][m] = best_v[m]; bis[wid][m] = best_i[m]; }
    }
    __syncthreads();
    if (tid < MB) {
      const int m = tid;
      float bv = bvs[0][m];
      int bi = bis[0][m];
      for (int ww = 1; ww < GEMV_WAVES; ++ww)
        if (better(bvs[ww][m], bis[ww][m], bv, bi)) { bv = bvs[ww][m]; bi = bis[ww][m]; }
      p.part_val[(size_t)m * gridDim.x + blockIdx.x] = bv;
      p.part_idx[(size_t)m * gridDim.x + blockIdx.x] = bi;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const uint32_t done = atomicAdd(p.counter, 1u);
      last = (done == gridDim.x - 1);
    }
    __syncthreads();
    if (last) {
      __threadfence();
      for (int m = 0; m < mcount; ++m) {
        float bv = 0.f;
        int bi = -1;
        for (int b = tid; b < (int)gridDim.x; b += GEMV_THREADS) {
          const float v = __builtin_nontemporal_load(p.part_val + (size_t)m * gridDim.x + b);
          const int i = __builtin_nontemporal_load(p.part_idx + (size_t)m * gridDim.x + b);
          if (better(v, i, bv, bi)) { bv = v; bi = i; }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ov = __shfl_xor(bv, o);
          const int oi = __shfl_xor(bi, o);
          if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
        }
        if (lane == 0) { bvs[wid][0] = bv; bis[wid][0] = bi; }
        __syncthreads();
        if (tid == 0) {
          for (int ww = 1; ww < GEMV_WAVES; ++ww)
            if (better(bvs[ww][0], bis[ww][0], bv, bi)) { bv = bvs[ww][0]; bi = bis[ww][0]; }
          if (p.next) p.next[m0 + m] = bi;
        }
        __syncthreads();
      }
      if (tid == 0) *p.counter = 0u;
    }
  }
}

// ------------------------------------------------------------------ launcher
static int cpl_for(int K) {
  const int c = (K / 8 + 63) / 64;
  if (c <= 1) return 1;
  if (c <= 2) return 2;
  if (c <= 4) return 4;
  if (c <= 6) return 6;
  if (c <= 8) return 8;
  return -1;
}

int gemv_logits_blocks(int N, int K) {
  const int cpl = cpl_for(K);
  const int rpw = cpl <= 2 ? 4 : 2;
  const int rows_per_group = GEMV_WAVES * rpw;
  const int groups = 8;
  return (N + rows_per_group * groups - 1) / (rows_per_group * groups);
}

template <typename W, int EPI, int MB, int CPL>
static hipError_t launch_gemv(GemvParams p, hipStream_t s) {
  constexpr int RPW = (CPL <= 2) ? 4 : 2;
  const int slots_total = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const int rows_per_group = GEMV_WAVES * RPW;
  int groups = 1;
  if (EPI == EPI_LOGITS) groups = 8;
  const int gx = (slots_total + rows_per_group * groups - 1) / (rows_per_group * groups);
  p.groups = groups;
  const int gy = (p.M + MB - 1) / MB;
  const size_t lds = (size_t)MB * p.K * sizeof(float) + MB * 4 * sizeof(float);
  gemv_kernel<W, EPI, MB, CPL, RPW><<<dim3(gx, gy), GEMV_THREADS, lds, s>>>(p);
  return hipGetLastError();
}

template <typename W, int EPI, int MB>
static hipError_t dispatch_cpl(GemvParams p, hipStream_t s) {
  switch (cpl_for(p.K)) {
    case 1: return launch_gemv<W, EPI, MB, 1>(p, s);
    case 2: return launch_gemv<W, EPI, MB, 2>(p, s);
    case 4: return launch_gemv<W, EPI, MB, 4>(p, s);
    case 6: return launch_gemv<W, EPI, MB, 6>(p, s);
    case 8: return launch_gemv<W, EPI, MB, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename W, int EPI>
static hipError_t dispatch_mb(GemvParams p, hipStream_t s) {
  if (p.M == 1) return dispatch_cpl<W, EPI, 1>(p, s);
  if (EPI == EPI_LOGITS && p.M > GEMV_LOGITS_MAX_M) return hipErrorInvalidValue;
  return dispatch_cpl<W, EPI, 4>(p, s);
}

hipError_t gemv(int dt, int epi, GemvParams p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.K % 8 != 0) return hipErrorInvalidValue;
  if (dt == DT_BF16) {
    switch (epi) {
      case EPI_STORE: return dispatch_mb<bf16, EPI_STORE>(p, s);
      case EPI_RESID: return dispatch_mb<bf16, EPI_RESID>(p, s);
      case EPI_SWIGLU: return dispatch_mb<bf16, EPI_SWIGLU>(p, s);
      case EPI_LOGITS: return dispatch_mb<bf16, EPI_LOGITS>(p, s);
    }
  } else {
    switch (epi) {
      case EPI_STORE: return dispatch_mb<float, EPI_STORE>(p, s);
      case EPI_RESID: return dispatch_mb<float, EPI_RESID>(p, s);
      case EPI_SWIGLU: return dispatch_mb<float, EPI_SWIGLU>(p, s);
      case EPI_LOGITS: return dispatch_mb<float, EPI_LOGITS>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fsk
