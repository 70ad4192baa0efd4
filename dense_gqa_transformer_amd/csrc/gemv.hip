// GEMV entry points: the bf16 / fp32 / int8 instantiations and the argmax of
// the lm_head's per-block bests (the fp8 instantiations are in gemv_f8.hip).
#include "gemv_impl.h"

namespace fsk {

// Final step of the LOGITS epilogue: one workgroup per row reduces the
// per-block (value, index) bests to the greedy ID.
__global__ __launch_bounds__(1024) void argmax_partials_kernel(const float* __restrict__ pv,
                                                               const int32_t* __restrict__ pi, int nblocks,
                                                               int32_t* __restrict__ next) {
  constexpr int NTH = 1024, PER = 16;       // a thread's partials of a stretch, requested together
  __shared__ float sv[NTH / 64];
  __shared__ int si[NTH / 64];
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const float* rv = pv + (size_t)m * nblocks;
  const int32_t* ri = pi + (size_t)m * nblocks;
  float bv = 0.f;
  int bi = -1;
  for (int base = 0; base < nblocks; base += NTH * PER) {
    float v[PER];
    int ix[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = min(base + tid + j * NTH, nblocks - 1);   // past the end: re-read, skipped
      v[j] = rv[c];
      ix[j] = ri[c];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (base + tid + j * NTH < nblocks && better(v[j], ix[j], bv, bi)) { bv = v[j]; bi = ix[j]; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (lane == 0) { sv[wid] = bv; si[wid] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int ww = 1; ww < NTH / 64; ++ww)
      if (better(sv[ww], si[ww], bv, bi)) { bv = sv[ww]; bi = si[ww]; }
    next[m] = bi;
  }
}

hipError_t argmax_partials(const float* pv, const int32_t* pi, int nblocks, int M, int32_t* next,
                           hipStream_t s) {
  if (M <= 0) return hipSuccess;
  argmax_partials_kernel<<<M, 1024, 0, s>>>(pv, pi, nblocks, next);
  return hipGetLastError();
}

int gemv_logits_blocks(int dt, int N, int K) {
  (void)K;
  const int rows_per_group = GEMV_WAVES * logits_rpw(dt == DT_I8 || dt == DT_F8);
  const int groups = GEMV_LOGITS_GROUPS;
  return (N + rows_per_group * groups - 1) / (rows_per_group * groups);
}

hipError_t gemv(int dt, int epi, GemvParams p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.K % 8 != 0) return hipErrorInvalidValue;
  if (p.aquant && (dt != DT_F8 || p.gamma == nullptr)) return hipErrorInvalidValue;
  if (dt == DT_F8) return gemv_f8(epi, p, s);
  if (dt == DT_I8) {
    if (p.K % 16 != 0 || p.wscale == nullptr) return hipErrorInvalidValue;
    switch (epi) {
      case EPI_STORE: return dispatch_mb<int8_t, EPI_STORE>(p, s);
      case EPI_RESID: return dispatch_mb<int8_t, EPI_RESID>(p, s);
      case EPI_SWIGLU: return dispatch_mb<int8_t, EPI_SWIGLU>(p, s);
      case EPI_LOGITS: return dispatch_mb<int8_t, EPI_LOGITS>(p, s);
    }
    return hipErrorInvalidValue;
  }
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
