// MFMA GEMM for few activation rows (M <= 64): batched decode steps and short
// prompts.
//
// C[M, N] = A[M, K] . B[N, K]^T as in gemm.hip (B a weight stored [out, in],
// "Coming back to Failed Star", First sitting, item 3), but shaped for the
// case where the weight, not the arithmetic, is the cost: a workgroup owns a
// slab of 32 * NT weight rows and every activation row, so each weight byte is
// fetched once.  The 4 waves split K four ways and stream their operands
// straight from global memory into MFMA fragments (no LDS staging); the four
// partial products meet in LDS for the epilogue.
//
// Fragments: for a 64-wide K chunk, lane l supplies row (l % 32) of its 32-row
// tile and the 32 consecutive k at 32 * (l / 32), eight per
// v_mfma_f32_32x32x16_bf16 step, identically for both operands, so each
// product sums every k of the chunk exactly once and each lane reads 64
// contiguous bytes of a row.  With the weight fragment as the first operand the
// 32x32 result holds (weight row 8*(r/4) + 4*(l/32) + r%4, activation row
// l%32) in register r.
#include "common.h"
#include "kernels.h"

namespace fsk {

namespace {

constexpr int SK_WAVES = 4;

template <int EPI, int NT, int MT, bool PIPE>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const bf16* __restrict__ A, int lda,
                                                          const bf16* __restrict__ A_lo,
                                                          const bf16* __restrict__ B, int ldb,
                                                          void* __restrict__ out, int ldc, int M, int N, int K,
                                                          const float* __restrict__ colscale) {
  constexpr int NS = 32 * NT;                 // weight rows (output columns) of this workgroup
  constexpr int MS = 32 * MT;                 // activation rows covered
  constexpr int RS = NS + 1;                  // padded LDS row: the partial sums of one activation row
  __shared__ float red[SK_WAVES][MS * RS];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * NS;
  const int m0 = blockIdx.z * MS;             // activation rows of this workgroup (split blockIdx.z)
  const int ks = K / (int)gridDim.y;          // K range of this workgroup (split blockIdx.y)
  const int kw = ks / SK_WAVES, kb = blockIdx.y * ks + wid * kw;

  const bf16* bp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) bp[t] = B + (size_t)min(n0 + 32 * t + r, N - 1) * ldb + kb + 32 * h;
  const bf16* ap[MT];
  const bf16* alp[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const size_t row = (size_t)min(m0 + 32 * i + r, M - 1);
    ap[i] = A + row * lda + kb + 32 * h;
    alp[i] = (A_lo != nullptr) ? A_lo + row * lda + kb + 32 * h : nullptr;
  }
  const bool lo = (A_lo != nullptr);

  f32x16 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][i][e] = 0.f;

  // One 64-wide K chunk's fragments.  PIPE (launches of a few hundred
  // workgroups, where each one's latency is the cost): two buffers ping-pong,
  // chunk c + 1 requested before chunk c's products in a loop body without
  // branches (the tail of one or two chunks is peeled), so that the
  // compiler's in-order load counting lets the two chunks overlap.  Otherwise
  // one buffer, fewer registers and more workgroups per CU.
  struct Frag {
    bf16x8 b[NT][4], a[MT][4], al[MT][4];
  };
  auto load = [&](int k, Frag& f) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) f.b[t][s] = *reinterpret_cast<const bf16x8*>(bp[t] + k + 8 * s);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s) f.a[i][s] = *reinterpret_cast<const bf16x8*>(ap[i] + k + 8 * s);
    if (lo) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s) f.al[i][s] = *reinterpret_cast<const bf16x8*>(alp[i] + k + 8 * s);
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          acc[t][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[t][s], f.a[i][s], acc[t][i], 0, 0, 0);
          if (lo) acc[t][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[t][s], f.al[i][s], acc[t][i], 0, 0, 0);
        }
  };
  const int nk = kw / 64;                      // >= 1 (K % (256 * splits) == 0)
  if constexpr (PIPE) {
    Frag fa, fb;
    load(0, fa);
    int c = 0;
    for (; c + 2 < nk; c += 2) {
      load(64 * (c + 1), fb);
      mma(fa);
      load(64 * (c + 2), fa);
      mma(fb);
    }
    if (c + 1 < nk) {
      load(64 * (c + 1), fb);
      mma(fa);
      mma(fb);
    } else {
      mma(fa);
    }
  } else {
    for (int c = 0; c < nk; ++c) {
      Frag f;
      load(64 * c, f);
      mma(f);
    }
  }

  // ---- the four K quarters meet in LDS: red[w][m * RS + n]
  float* R = red[wid];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int n = 32 * t + 8 * (e >> 2) + 4 * h + (e & 3);
        R[(32 * i + r) * RS + n] = acc[t][i][e];
      }
  __syncthreads();

  const int rows = min(M - m0, MS);
  if (EPI == GEPI_SWIGLU_BF16) {
    // the slab is one packed [32 gate | 32 up] block: 32 output features
    const int f0 = n0 / 2;
    for (int idx = threadIdx.x; idx < rows * 32; idx += 256) {
      const int m = idx >> 5, n = idx & 31;
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < SK_WAVES; ++w) {
        g += red[w][m * RS + n];
        u += red[w][m * RS + 32 + n];
      }
      if (colscale != nullptr) {
        g *= colscale[n0 + n];
        u *= colscale[n0 + 32 + n];
      }
      reinterpret_cast<bf16*>(out)[(size_t)(m0 + m) * ldc + f0 + n] = (bf16)(silu(g) * u);
    }
  } else {
    for (int idx = threadIdx.x; idx < rows * NS; idx += 256) {
      const int m = idx / NS, n = idx % NS;
      if (n0 + n >= N) continue;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < SK_WAVES; ++w) v += red[w][m * RS + n];
      if (colscale != nullptr) v *= colscale[n0 + n];
      const size_t o = (size_t)(m0 + m) * ldc + n0 + n;
      if (EPI == GEPI_STORE_BF16) reinterpret_cast<bf16*>(out)[o] = (bf16)v;
      else if (EPI == GEPI_STORE_F32) reinterpret_cast<float*>(out)[o] = v;
      else if (EPI == GEPI_PART_F32) reinterpret_cast<float*>(out)[(size_t)blockIdx.y * M * ldc + o] = v;
      else reinterpret_cast<float*>(out)[o] += v;
    }
  }
}

template <int EPI, int NT>
hipError_t launch_nt(const bf16* a, int lda, const bf16* alo, const bf16* b, int ldb, void* out, int ldc, int M,
                     int N, int K, const float* cs, int ksplit, hipStream_t s) {
  // SwiGLU with more than 32 rows: 32-row halves in separate workgroups (each
  // streams the weight slab once more, in exchange for twice the workgroups:
  // N / 64 slabs alone leave most CUs idle)
  if (EPI == GEPI_SWIGLU_BF16 && M > 32 && ksplit == 1) {
    const dim3 g2((N + 32 * NT - 1) / (32 * NT), 1, (M + 31) / 32);
    const bool pipe2 = (long long)g2.x * g2.z <= 512;
    if (pipe2) gemm_skinny_kernel<EPI, NT, 1, true><<<g2, 256, 0, s>>>(a, lda, alo, b, ldb, out, ldc, M, N, K, cs);
    else gemm_skinny_kernel<EPI, NT, 1, false><<<g2, 256, 0, s>>>(a, lda, alo, b, ldb, out, ldc, M, N, K, cs);
    return hipGetLastError();
  }
  const dim3 grid((N + 32 * NT - 1) / (32 * NT), ksplit);
  const bool pipe = (long long)grid.x * grid.y <= 512;
  if (M <= 32) {
    if (pipe) gemm_skinny_kernel<EPI, NT, 1, true><<<grid, 256, 0, s>>>(a, lda, alo, b, ldb, out, ldc, M, N, K, cs);
    else gemm_skinny_kernel<EPI, NT, 1, false><<<grid, 256, 0, s>>>(a, lda, alo, b, ldb, out, ldc, M, N, K, cs);
  } else {
    if (pipe) gemm_skinny_kernel<EPI, NT, 2, true><<<grid, 256, 0, s>>>(a, lda, alo, b, ldb, out, ldc, M, N, K, cs);
    else gemm_skinny_kernel<EPI, NT, 2, false><<<grid, 256, 0, s>>>(a, lda, alo, b, ldb, out, ldc, M, N, K, cs);
  }
  return hipGetLastError();
}

}  // namespace

bool gemm_skinny_ok(int epi, const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                    const void* A_lo) {
  if (M <= 0 || M > 64 || N <= 0 || K <= 0 || K % 256 != 0 || N % 32 != 0) return false;
  if (epi == GEPI_SWIGLU_BF16 && N % 64 != 0) return false;
  if (lda % 8 || ldb % 8) return false;
  const uintptr_t al = (uintptr_t)A | (uintptr_t)B | (uintptr_t)A_lo;
  return (al & 15) == 0;
}

hipError_t gemm_skinny(int epi, const void* A, int lda, const void* B, int ldb, void* out, int ldc, int M, int N,
                       int K, hipStream_t s, const void* A_lo, const float* colscale, int ksplit) {
  if (ksplit < 1 || (ksplit > 1 && epi != GEPI_PART_F32) || K % (256 * ksplit) != 0) return hipErrorInvalidValue;
  const bf16* a = (const bf16*)A;
  const bf16* b = (const bf16*)B;
  const bf16* al = (const bf16*)A_lo;
  const float* cs = colscale;
  switch (epi) {
    case GEPI_STORE_BF16: return launch_nt<GEPI_STORE_BF16, 1>(a, lda, al, b, ldb, out, ldc, M, N, K, cs, 1, s);
    case GEPI_STORE_F32:
      // very wide outputs (the tied head): 64 weight rows per workgroup, so each
      // streams 128 KB rather than 64 KB per launch share
      if (N >= 65536 && N % 64 == 0)
        return launch_nt<GEPI_STORE_F32, 2>(a, lda, al, b, ldb, out, ldc, M, N, K, cs, 1, s);
      return launch_nt<GEPI_STORE_F32, 1>(a, lda, al, b, ldb, out, ldc, M, N, K, cs, 1, s);
    case GEPI_RESID_F32: return launch_nt<GEPI_RESID_F32, 1>(a, lda, al, b, ldb, out, ldc, M, N, K, cs, 1, s);
    case GEPI_PART_F32: return launch_nt<GEPI_PART_F32, 1>(a, lda, al, b, ldb, out, ldc, M, N, K, cs, ksplit, s);
    case GEPI_SWIGLU_BF16: return launch_nt<GEPI_SWIGLU_BF16, 2>(a, lda, al, b, ldb, out, ldc, M, N, K, cs, 1, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fsk
