// bf16 MFMA GEMM for the prefill projections and MLP (the dense contractions).
//
// C[M, N] = A[M, K] . B[N, K]^T: A holds activation rows, B a weight stored
// [out, in] ("Coming back to Failed Star", First sitting, item 3), so both
// operands are K-contiguous.  fp32 accumulation in v_mfma_f32_32x32x16_bf16.
//
// Tiling: 128x128 output tile per workgroup of 4 waves (2x2, 64x64 per wave =
// 2x2 MFMA blocks), K step 64, double-buffered LDS with rows padded by 16 B
// so that the 128-bit fragment reads are bank-conflict free.  One barrier per
// K step: the next tile's global loads are issued before the MFMAs of the
// current one and written to the other LDS buffer after them.
//
// Fragment layout: lane l supplies row (l % 32) of its 32-row block and the
// 8 consecutive k at 8*(l/32) of the 16-wide step, identically for A and B,
// so the product sums over the same k whatever order the unit uses.  The
// 32x32 result holds element (8*(r/4) + 4*(l/32) + r%4, l%32) in register r.
#include "common.h"
#include "kernels.h"

namespace fsk {

static constexpr int BM = 128, BN = 128, BK = 64;
static constexpr int LDK = BK + 8;   // padded row length (elements)

template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const bf16* __restrict__ A, int lda,
                                                        const bf16* __restrict__ B, int ldb,
                                                        void* __restrict__ out, int ldc,
                                                        int M, int N, int K,
                                                        const bf16* __restrict__ A_lo,
                                                        const float* __restrict__ colscale) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;

  // global -> register staging: 4 x 16 B of A and of B per thread
  u32x4 ra[4], rb[4];
  // K steps [0, nk0) read A; with A_lo, steps [nk0, 2*nk0) read A_lo against the same B
  const int nk0 = K / BK;
  auto gload = [&](int kt) {
    const bf16* a = (kt < nk0) ? A : A_lo;
    const int k0 = (kt < nk0 ? kt : kt - nk0) * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int r = id >> 3, c8 = (id & 7) * 8;
      const int gm = m0 + r, gn = n0 + r;
      ra[i] = (gm < M) ? *reinterpret_cast<const u32x4*>(a + (size_t)gm * lda + k0 + c8) : u32x4{0, 0, 0, 0};
      rb[i] = (gn < N) ? *reinterpret_cast<const u32x4*>(B + (size_t)gn * ldb + k0 + c8) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int r = id >> 3, c8 = (id & 7) * 8;
      *reinterpret_cast<u32x4*>(&As[buf][r * LDK + c8]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][r * LDK + c8]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (A_lo != nullptr) ? 2 * nk0 : nk0;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm * 64 + i * 32 + lrow) * LDK + kk + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn * 64 + j * 32 + lrow) * LDK + kk + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const int col_in = lane & 31, rq = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + rq + (r & 3);
      if (row >= M) continue;
      if (EPI == GEPI_SWIGLU_BF16) {
        // the wave's 64 columns are [32 gate | matching 32 up] of the packed matrix
        if (n0 + wn * 64 >= N) continue;
        const int f = (n0 + wn * 64) / 2 + col_in;
        float g = acc[i][0][r], u = acc[i][1][r];
        if (colscale != nullptr) {
          g *= colscale[n0 + wn * 64 + col_in];
          u *= colscale[n0 + wn * 64 + 32 + col_in];
        }
        reinterpret_cast<bf16*>(out)[(size_t)row * ldc + f] = (bf16)(silu(g) * u);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 64 + j * 32 + col_in;
          if (col >= N) continue;
          const size_t o = (size_t)row * ldc + col;
          const float v = colscale != nullptr ? acc[i][j][r] * colscale[col] : acc[i][j][r];
          if (EPI == GEPI_STORE_BF16) reinterpret_cast<bf16*>(out)[o] = (bf16)v;
          else if (EPI == GEPI_STORE_F32) reinterpret_cast<float*>(out)[o] = v;
          else reinterpret_cast<float*>(out)[o] += v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large-M variant: 256x256 tile, 8 waves (2 x 4), 128x64 per wave = 4x2 MFMA
// blocks, so each 16-wide K step reads 6 fragments from LDS for 8 MFMAs (vs 4
// for 4 in the 128x128 tile) and every A / B element fetched from L2 serves
// twice as many products.  Workgroups are renumbered so that the tiles handed
// to one XCD (the hardware deals workgroups round-robin over the 8 XCDs) form
// a contiguous band that shares A and B tiles in that XCD's L2.
static constexpr int BM2 = 256, BN2 = 256;

template <int EPI>
__global__ __launch_bounds__(512) void gemm_bf16_big_kernel(const bf16* __restrict__ A, int lda,
                                                            const bf16* __restrict__ B, int ldb,
                                                            void* __restrict__ out, int ldc,
                                                            int M, int N, int K, const bf16* __restrict__ A_lo,
                                                            int tiles_n, int nblocks,
                                                            const float* __restrict__ colscale) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM2 * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN2 * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 2, wn = wid & 3;
  // XCD-aware renumbering (exact when nblocks % 8 == 0, identity otherwise)
  int bid = blockIdx.x;
  if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
  const int n0 = (bid % tiles_n) * BN2, m0 = (bid / tiles_n) * BM2;

  const int nk0 = K / BK;
  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const bf16* a = (kt < nk0) ? A : A_lo;
    const int k0 = (kt < nk0 ? kt : kt - nk0) * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 512 * i;
      const int r = id >> 3, c8 = (id & 7) * 8;
      const int gm = m0 + r, gn = n0 + r;
      ra[i] = (gm < M) ? *reinterpret_cast<const u32x4*>(a + (size_t)gm * lda + k0 + c8) : u32x4{0, 0, 0, 0};
      rb[i] = (gn < N) ? *reinterpret_cast<const u32x4*>(B + (size_t)gn * ldb + k0 + c8) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 512 * i;
      const int r = id >> 3, c8 = (id & 7) * 8;
      *reinterpret_cast<u32x4*>(&As[buf][r * LDK + c8]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][r * LDK + c8]) = rb[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (A_lo != nullptr) ? 2 * nk0 : nk0;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][(wm * 128 + i * 32 + lrow) * LDK + kk + lk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][(wn * 64 + j * 32 + lrow) * LDK + kk + lk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  const int col_in = lane & 31, rq = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + rq + (r & 3);
      if (row >= M) continue;
      if (EPI == GEPI_SWIGLU_BF16) {
        if (n0 + wn * 64 >= N) continue;
        const int f = (n0 + wn * 64) / 2 + col_in;
        float g = acc[i][0][r], u = acc[i][1][r];
        if (colscale != nullptr) {
          g *= colscale[n0 + wn * 64 + col_in];
          u *= colscale[n0 + wn * 64 + 32 + col_in];
        }
        reinterpret_cast<bf16*>(out)[(size_t)row * ldc + f] = (bf16)(silu(g) * u);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 64 + j * 32 + col_in;
          if (col >= N) continue;
          const size_t o = (size_t)row * ldc + col;
          const float v = colscale != nullptr ? acc[i][j][r] * colscale[col] : acc[i][j][r];
          if (EPI == GEPI_STORE_BF16) reinterpret_cast<bf16*>(out)[o] = (bf16)v;
          else if (EPI == GEPI_STORE_F32) reinterpret_cast<float*>(out)[o] = v;
          else reinterpret_cast<float*>(out)[o] += v;
        }
      }
    }
  }
}

template <int EPI>
static void launch_big(const bf16* a, int lda, const bf16* b, int ldb, void* out, int ldc, int M, int N, int K,
                       const bf16* alo, const float* cs, hipStream_t s) {
  const int tn = (N + BN2 - 1) / BN2, tm = (M + BM2 - 1) / BM2;
  gemm_bf16_big_kernel<EPI><<<tn * tm, 512, 0, s>>>(a, lda, b, ldb, out, ldc, M, N, K, alo, tn, tn * tm, cs);
}

hipError_t gemm_bf16(int epi, const void* A, int lda, const void* B, int ldb, void* out, int ldc,
                     int M, int N, int K, hipStream_t s, const void* A_lo, const float* colscale) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % BK != 0) return hipErrorInvalidValue;
  if (epi == GEPI_SWIGLU_BF16 && N % 64 != 0) return hipErrorInvalidValue;
  if (gemm_skinny_ok(epi, A, lda, B, ldb, M, N, K, A_lo))
    return gemm_skinny(epi, A, lda, B, ldb, out, ldc, M, N, K, s, A_lo, colscale);
  if (gemm_dma_ok(epi, A, lda, B, ldb, out, ldc, M, N, K, A_lo))
    return gemm_dma(epi, A, lda, B, ldb, out, ldc, M, N, K, s, A_lo, colscale);
  const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  const bf16* a = (const bf16*)A;
  const bf16* b = (const bf16*)B;
  const bf16* alo = (const bf16*)A_lo;
  // large problems: 256x256 tiles once there are enough of them to fill the chip
  if (M >= 1024 && (long long)((M + BM2 - 1) / BM2) * ((N + BN2 - 1) / BN2) >= 256) {
    switch (epi) {
      case GEPI_STORE_BF16: launch_big<GEPI_STORE_BF16>(a, lda, b, ldb, out, ldc, M, N, K, alo, colscale, s); break;
      case GEPI_RESID_F32: launch_big<GEPI_RESID_F32>(a, lda, b, ldb, out, ldc, M, N, K, alo, colscale, s); break;
      case GEPI_SWIGLU_BF16: launch_big<GEPI_SWIGLU_BF16>(a, lda, b, ldb, out, ldc, M, N, K, alo, colscale, s); break;
      case GEPI_STORE_F32: launch_big<GEPI_STORE_F32>(a, lda, b, ldb, out, ldc, M, N, K, alo, colscale, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (epi) {
    case GEPI_STORE_BF16: gemm_bf16_kernel<GEPI_STORE_BF16><<<grid, 256, 0, s>>>(a, lda, b, ldb, out, ldc, M, N, K, (const bf16*)A_lo, colscale); break;
    case GEPI_RESID_F32: gemm_bf16_kernel<GEPI_RESID_F32><<<grid, 256, 0, s>>>(a, lda, b, ldb, out, ldc, M, N, K, (const bf16*)A_lo, colscale); break;
    case GEPI_SWIGLU_BF16: gemm_bf16_kernel<GEPI_SWIGLU_BF16><<<grid, 256, 0, s>>>(a, lda, b, ldb, out, ldc, M, N, K, (const bf16*)A_lo, colscale); break;
    case GEPI_STORE_F32: gemm_bf16_kernel<GEPI_STORE_F32><<<grid, 256, 0, s>>>(a, lda, b, ldb, out, ldc, M, N, K, (const bf16*)A_lo, colscale); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fsk
