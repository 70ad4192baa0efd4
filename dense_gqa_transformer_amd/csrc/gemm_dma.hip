// Large bf16 MFMA GEMM for the prefill projections and MLP: 256x256 output
// tile per workgroup of 8 waves, two per SIMD (2 x 4, 128x64 per wave = 4x2
// blocks of v_mfma_f32_32x32x16_bf16), operands streamed from HBM straight
// into LDS.  Two waves per SIMD let one wave's waits for the stage barrier
// overlap the other's products (measured 3-8% faster than one wave of 128x128
// per SIMD on the four prefill shapes).
//
// C[M, N] = A[M, K] . B[N, K]^T with both operands K-contiguous: A holds
// activation rows, B a weight stored [out, in] ("Coming back to Failed Star",
// First sitting, item 3).  fp32 accumulation.
//
// Pipeline.  K is consumed in stages of 32.  Each stage's A and B tiles
// (2 x 16 KB) are fetched with global_load_lds (16 B per lane, the 64 lanes of
// one instruction fill 1 KB of LDS contiguously), so no VGPR staging and no
// ds_write instructions are spent on them.  Five stage buffers (all 160 KB of
// LDS) form a ring: while the waves multiply stage k, stages k+1..k+4 are in
// flight.  The buffers are five distinct LDS objects and the K loop is
// unrolled by five, so every access names its buffer statically; the copies
// are written out (dma16), so the compiler adds no waits for them, and the one
// wait per stage is the explicit vmcnt(12) (this wave's four loads for stage
// k+1 done) before the stage's single barrier.
// Measured limits (standalone, four prefill shapes): with the fills removed
// the loop reaches 50-58% of the bf16 peak, barriers cost under 1%; the
// fragment reads plus the DMA writes ask about as many LDS bytes per stage as
// the matrix unit has cycles, which bounds this design.
//
// Bank conflicts.  A stage row is 32 bf16 = 64 B (four 16-B chunks).  Row R
// stores its k-chunk c at chunk slot c ^ ((R >> 2) & 3): the 16 rows a
// quarter-wave fragment read touches then cover all 64 banks once.  The DMA
// side picks, for each LDS slot, the global chunk that belongs there.
//
// Fragments.  MFMA operand "A" is the weight fragment and operand "B" the
// activation fragment, so lane l of a 32x32 result holds activation row
// (l % 32) and four consecutive output columns 8*(r/4) + 4*(l/32) + (0..3) in
// registers r..r+3.  The epilogue writes those quads into LDS (reused once the
// K loop has drained) with an XOR-swizzled row layout and streams whole rows
// back to HBM in 16-B chunks.
#include "gemm_dma_common.h"

namespace fsk {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// The 8-bit exponent (E8M0) of a power-of-two fp32 scale: its exponent field
// (0, i.e. 2^-127, for a zero scale, whose codes are all zero).
__device__ __forceinline__ int e8m0(float sc) { return (int)((__float_as_uint(sc) >> 23) & 0xFFu); }

template <int EPI, bool LO8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma_kernel(const bf16* __restrict__ A, int lda, const bf16* __restrict__ A_lo,
                  const bf16* __restrict__ B, int ldb, void* __restrict__ out, int ldc,
                  int M, int N, int K, int tiles_n, int nblocks, int gm, const float* __restrict__ colscale,
                  const RopeKvParams rp, const Lo8Params l8) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;
  int m0, n0;
  tile_origin(nblocks, tiles_n, gm, m0, n0);

  // DMA assignment: wave w, instruction j fills tile rows (2w + j)*16 + lane/4
  // (chunk slot lane % 4) of A and of B.  Rows past M / N re-read the last
  // valid row; their results are never stored.
  const int lr = lane >> 2;
  const int kc = (lane & 3) ^ ((lr >> 2) & 3);
  const bf16* pa[2];
  const bf16* pl[2];
  const bf16* pb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ra = min(m0 + wid * 32 + j * 16 + lr, M - 1);
    const int rb = min(n0 + wid * 32 + j * 16 + lr, N - 1);
    pa[j] = A + (size_t)ra * lda + kc * 8;
    pl[j] = (A_lo != nullptr ? A_lo : A) + (size_t)ra * lda + kc * 8;
    pb[j] = B + (size_t)rb * ldb + kc * 8;
  }
  const int nk0 = K / DK;
  const int nk = (A_lo != nullptr) ? 2 * nk0 : nk0;
  const uint8_t* pa8[2];
  const uint8_t* pb8[2];
  if constexpr (LO8) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ra = min(m0 + wid * 32 + j * 16 + lr, M - 1);
      const int rb = min(n0 + wid * 32 + j * 16 + lr, N - 1);
      pa8[j] = l8.a + (size_t)ra * K + kc * 16;
      pb8[j] = l8.b + (size_t)rb * K + kc * 16;
    }
  }

  auto issue = [&](auto Sc, int st) {
    bf16* L = stage_buf<decltype(Sc)::value>();
    const bool lo = st >= nk0;
    const int k0 = (lo ? st - nk0 : st) * DK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dma16((lo ? pl[j] : pa[j]) + k0, L + (wid * 2 + j) * 16 * DK);
      dma16(pb[j] + k0, L + TILE * DK + (wid * 2 + j) * 16 * DK);
    }
  };

  const int lrow = lane & 31;
  const int sw = (lrow >> 2) & 3;
  const int aoff = (wm * 128 + lrow) * DK, boff = TILE * DK + (wn * 64 + lrow) * DK;
  const int so0 = ((lane >> 5) ^ sw) * 8, so1 = ((2 + (lane >> 5)) ^ sw) * 8;
  // fragment set `set` of block i is dwords [4 set, 4 set + 4) of fa8[i] (fb8
  // for the weight blocks): the two sets of one stage are then the 32 bytes of
  // an fp8 operand as they stand, with no register copies
  i32x8 fa8[4], fb8[2];
  auto fread = [&](auto Sc, int set, int q) {
    const bf16* L = stage_buf<decltype(Sc)::value>();
    const int so = q ? so1 : so0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(L + aoff + i * 32 * DK + so);
#pragma unroll
      for (int e = 0; e < 4; ++e) fa8[i][4 * set + e] = v[e];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(L + boff + j * 32 * DK + so);
#pragma unroll
      for (int e = 0; e < 4; ++e) fb8[j][4 * set + e] = v[e];
    }
  };
  auto half = [](const i32x8& f, int set) {
    const i32x4 h = set ? i32x4{f[4], f[5], f[6], f[7]} : i32x4{f[0], f[1], f[2], f[3]};
    return __builtin_bit_cast(bf16x8, h);
  };
  f32x16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;
  auto mm = [&](int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(half(fb8[j], set), half(fa8[i], set), acc[j][i], 0, 0, 0);
  };
  // An fp8 remainder stage: the two fragment sets hold the stage's two 16-B
  // chunks per lane (logical chunks l/32 and 2 + l/32 of the row), which make
  // the 32 codes of one v_mfma_scale_f32_32x32x64_f8f6f4 operand; the row
  // scales of the remainder (activation rows) and of the weights' fp8 copy
  // enter as the instruction's per-lane 8-bit exponents, so the product lands
  // in the fp32 tile already scaled.
  int sa8[4] = {127, 127, 127, 127}, sb8[2] = {127, 127};
  if constexpr (LO8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sa8[i] = e8m0(l8.as[min(m0 + wm * 128 + i * 32 + lrow, M - 1)]);
#pragma unroll
    for (int j = 0; j < 2; ++j) sb8[j] = e8m0(l8.bs[min(n0 + wn * 64 + j * 32 + lrow, N - 1)]);
  }
  auto mm8 = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb8[j], fa8[i], acc[j][i], 0, 0, 0, sb8[j], 0,
                                                                    sa8[i]);
  };

  if constexpr (LO8) {
    // Per 64 K values: two bf16 stages (value) and one fp8 stage (remainder),
    // so stage kt's type is kt % 3 and its ring buffer kt % 5, both static in
    // a loop unrolled by 15.  A stage past the end re-reads the last 64 K
    // values in the type its position calls for (never multiplied).
    const int n64 = K / 64;
    const int nk8 = 3 * n64;
    auto issue8 = [&](auto Sc, auto Tc, int st) {
      constexpr int T = decltype(Tc)::value;
      bf16* L = stage_buf<decltype(Sc)::value>();
      const int c = min(st / 3, n64 - 1);
      if constexpr (T == 2) {
        char* L8 = reinterpret_cast<char*>(L);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          dma16(pa8[j] + c * 64, L8 + (wid * 2 + j) * 1024);
          dma16(pb8[j] + c * 64, L8 + TILE * 64 + (wid * 2 + j) * 1024);
        }
      } else {
        const int k0 = c * 64 + T * DK;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          dma16(pa[j] + k0, L + (wid * 2 + j) * 16 * DK);
          dma16(pb[j] + k0, L + TILE * DK + (wid * 2 + j) * 16 * DK);
        }
      }
    };
    issue8(Ic<0>{}, Ic<0>{}, 0);
    issue8(Ic<1>{}, Ic<1>{}, 1);
    issue8(Ic<2>{}, Ic<2>{}, 2);
    issue8(Ic<3>{}, Ic<0>{}, 3);
    __builtin_amdgcn_s_waitcnt(WAIT_VM12_LGKM0);
    lds_barrier();
    fread(Ic<0>{}, 0, 0);
    auto step8 = [&](auto Cc, auto Tc, int kt) {
      constexpr int C = decltype(Cc)::value, T = decltype(Tc)::value;
      issue8(Ic<(C + 4) % 5>{}, Ic<(T + 4) % 3>{}, kt + 4);
      fread(Ic<C>{}, 1, 1);
      if constexpr (T == 2) {
        mm8();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_s_waitcnt(WAIT_VM12_LGKM0);
        lds_barrier();
        fread(Ic<(C + 1) % 5>{}, 0, 0);
      } else {
        mm(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_s_waitcnt(WAIT_VM12_LGKM0);
        lds_barrier();
        fread(Ic<(C + 1) % 5>{}, 0, 0);
        mm(1);
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    };
    for (int kt = 0; kt < nk8; kt += 15) {
      step8(Ic<0>{}, Ic<0>{}, kt);
      step8(Ic<1>{}, Ic<1>{}, kt + 1);
      step8(Ic<2>{}, Ic<2>{}, kt + 2);
      if (kt + 3 >= nk8) break;
      step8(Ic<3>{}, Ic<0>{}, kt + 3);
      step8(Ic<4>{}, Ic<1>{}, kt + 4);
      step8(Ic<0>{}, Ic<2>{}, kt + 5);
      if (kt + 6 >= nk8) break;
      step8(Ic<1>{}, Ic<0>{}, kt + 6);
      step8(Ic<2>{}, Ic<1>{}, kt + 7);
      step8(Ic<3>{}, Ic<2>{}, kt + 8);
      if (kt + 9 >= nk8) break;
      step8(Ic<4>{}, Ic<0>{}, kt + 9);
      step8(Ic<0>{}, Ic<1>{}, kt + 10);
      step8(Ic<1>{}, Ic<2>{}, kt + 11);
      if (kt + 12 >= nk8) break;
      step8(Ic<2>{}, Ic<0>{}, kt + 12);
      step8(Ic<3>{}, Ic<1>{}, kt + 13);
      step8(Ic<4>{}, Ic<2>{}, kt + 14);
    }
  } else {
    // One stage: the loads of stage kt+4 (into the buffer read in stage kt-1),
    // then the two 16-wide K halves; the second half's fragments come from the
    // next stage, read after the barrier that publishes it.  Past the end the
    // ring re-reads the last stage into buffers nobody reads again, which keeps
    // the vmcnt bookkeeping uniform.
    issue(Ic<0>{}, 0);
    issue(Ic<1>{}, min(1, nk - 1));
    issue(Ic<2>{}, min(2, nk - 1));
    issue(Ic<3>{}, min(3, nk - 1));
    __builtin_amdgcn_s_waitcnt(WAIT_VM12_LGKM0);
    lds_barrier();
    fread(Ic<0>{}, 0, 0);

    auto step = [&](auto Cc, int kt) {
      constexpr int C = decltype(Cc)::value;
      issue(Ic<(C + 4) % 5>{}, min(kt + 4, nk - 1));
      fread(Ic<C>{}, 1, 1);
      mm(0);
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_s_waitcnt(WAIT_VM12_LGKM0);
      lds_barrier();
      fread(Ic<(C + 1) % 5>{}, 0, 0);
      mm(1);
  #pragma unroll
      for (int i = 0; i < 6; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
    for (int kt = 0; kt < nk; kt += 5) {
      step(Ic<0>{}, kt);
      if (kt + 1 >= nk) break;
      step(Ic<1>{}, kt + 1);
      if (kt + 2 >= nk) break;
      step(Ic<2>{}, kt + 2);
      if (kt + 3 >= nk) break;
      step(Ic<3>{}, kt + 3);
      if (kt + 4 >= nk) break;
      step(Ic<4>{}, kt + 4);
    }
  }

  // ---- epilogue: drain the ring, then each wave stages its 128x64 block in
  // its own 16 KB of LDS and writes whole rows.
  __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
  lds_barrier();
  if constexpr (EPI == GEPI_QKV_ROPE) {
    // (kept inline: through the shared epilogue the compiler spills here)
    if (colscale != nullptr) {
      const int hl = lane >> 5, ncol0 = n0 + wn * 64;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = min(ncol0 + 32 * j + 8 * g + 4 * hl, N - 4);
          const f32x4 sc = *reinterpret_cast<const f32x4*>(colscale + n);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][i][4 * g + e] *= sc[e];
        }
    }
    qkv_rope_epilogue(rp, acc, m0, n0, M, tid);
  } else {
    dma_epilogue<EPI>(acc, tid, m0, n0, M, N, out, ldc, colscale, nullptr, rp);
  }
}

// Usable when K is a multiple of 128, rows are 16-B aligned and the problem
// has enough 256x256 tiles to fill the chip; otherwise the caller picks
// another kernel.
bool gemm_dma_ok(int epi, const void* A, int lda, const void* B, int ldb, const void* out, int ldc,
                 int M, int N, int K, const void* A_lo) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || N % 8 != 0) return false;
  if (lda % 8 || ldb % 8 || ldc % 8) return false;
  const uintptr_t al = (uintptr_t)A | (uintptr_t)B | (uintptr_t)out | (uintptr_t)A_lo;
  if (al & 15) return false;
  if (epi == GEPI_SWIGLU_BF16 && N % 64 != 0) return false;
  const long long tiles = (long long)((M + TILE - 1) / TILE) * ((N + TILE - 1) / TILE);
  return M >= 1024 && tiles >= 256;
}

bool gemm_dma_rope_ok(const RopeKvParams& r, int M, int N) {
  return r.d == 128 && r.rot == 128 && !r.gated && r.nq % 2 == 0 && r.nkv % 2 == 0 && r.T == M &&
         r.S_per > 0 && M % r.S_per == 0 && N == (r.nq + 2 * r.nkv) * 128 && r.in_dt == DT_F32 &&
         r.q_dt == DT_BF16 && r.kv_dt == DT_BF16;
}

hipError_t gemm_dma(int epi, const void* A, int lda, const void* B, int ldb, void* out, int ldc,
                    int M, int N, int K, hipStream_t s, const void* A_lo, const float* colscale,
                    const RopeKvParams* rope, const Lo8Params* lo8) {
  if (colscale != nullptr && ((uintptr_t)colscale & 15)) return hipErrorInvalidValue;
  Lo8Params l8{};
  if (lo8 != nullptr) {
    l8 = *lo8;
    if (A_lo != nullptr || K % 64 != 0 || l8.a == nullptr || l8.b == nullptr || l8.as == nullptr ||
        l8.bs == nullptr || (((uintptr_t)l8.a | (uintptr_t)l8.b) & 15))
      return hipErrorInvalidValue;
  }
  RopeKvParams rp{};
  if (epi == GEPI_QKV_ROPE) {
    if (rope == nullptr || !gemm_dma_rope_ok(*rope, M, N)) return hipErrorInvalidValue;
    rp = *rope;
  }
  const int tn = (N + TILE - 1) / TILE, tm = (M + TILE - 1) / TILE;
  const int nb = tn * tm;
  const int gm = gemm_tile_group();
  const bf16* a = (const bf16*)A;
  const bf16* b = (const bf16*)B;
  const bf16* al = (const bf16*)A_lo;
  if (lo8 != nullptr) {
    switch (epi) {
      case GEPI_SWIGLU_BF16:
        gemm_dma_kernel<GEPI_SWIGLU_BF16, true><<<nb, 512, 0, s>>>(a, lda, nullptr, b, ldb, out, ldc, M, N, K, tn, nb, gm, colscale, rp, l8);
        break;
      case GEPI_STORE_F32:
        gemm_dma_kernel<GEPI_STORE_F32, true><<<nb, 512, 0, s>>>(a, lda, nullptr, b, ldb, out, ldc, M, N, K, tn, nb, gm, colscale, rp, l8);
        break;
      case GEPI_QKV_ROPE:
        gemm_dma_kernel<GEPI_QKV_ROPE, true><<<nb, 512, 0, s>>>(a, lda, nullptr, b, ldb, out, ldc, M, N, K, tn, nb, gm, colscale, rp, l8);
        break;
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (epi) {
    case GEPI_STORE_BF16:
      gemm_dma_kernel<GEPI_STORE_BF16, false><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, gm, colscale, rp, l8);
      break;
    case GEPI_RESID_F32:
      gemm_dma_kernel<GEPI_RESID_F32, false><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, gm, colscale, rp, l8);
      break;
    case GEPI_SWIGLU_BF16:
      gemm_dma_kernel<GEPI_SWIGLU_BF16, false><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, gm, colscale, rp, l8);
      break;
    case GEPI_STORE_F32:
      gemm_dma_kernel<GEPI_STORE_F32, false><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, gm, colscale, rp, l8);
      break;
    case GEPI_QKV_ROPE:
      gemm_dma_kernel<GEPI_QKV_ROPE, false><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, gm, colscale, rp, l8);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fsk
