// Large fp8 (e4m3) MFMA GEMM for the prefill projections of the fp8 weight
// option: the Q/K/V and gate/up products, whose inputs are the quantized norm
// outputs, so both operands are e4m3 codes with one power-of-two scale per
// row.
//
// C[M, N] = diag(rowscale) . (A[M, K] . B[N, K]^T) . diag(colscale), A and B
// K-contiguous code matrices (lda, ldb in bytes), fp32 accumulation.  Each
// product of two e4m3 values is exact in fp32, the power-of-two scales are
// exact factors, so the result is the oracle's sum of (code * scale)
// products up to the order of the fp32 additions.
//
// Same tiling, ring and epilogues as the bf16 kernel (gemm_dma_common.h): a
// stage row is 64 B, here 64 K values, so a stage carries twice the K of a
// bf16 stage for the same LDS bytes, and one v_mfma_scale_f32_32x32x64_f8f6f4
// per 32x32 block and stage does twice the bf16 instruction's work in twice
// its cycles.  The LDS traffic per matrix-unit cycle is the bf16 kernel's; the
// flops per stage double.
//
// Fragments.  Lane l of a 32x32x64 operand holds 32 values of row l % 32.  It
// takes the row's logical 16-B chunks (l / 32) and 2 + (l / 32) of the stage
// (two ds_read_b128, the same two reads a bf16 stage's two K halves use), so
// the four chunks of a row are spread over the two half-waves once; A and B
// lanes use the same assignment, which is all a dot product over K needs.
// The instruction's own 8-bit exponent scales are left at 2^0: the row scales
// are applied in the epilogue, in fp32, which is exact for powers of two.
//
// Pipeline.  The fragments of a whole stage live in registers (two sets,
// alternating), so a stage's barrier is followed by the reads of the next
// stage and the eight products of the current one, which overlap; the ring
// is reloaded one stage behind the barrier (all waves have read the stage
// whose buffer is refilled).
#include "gemm_dma_common.h"

namespace fsk {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int KS8 = 64;                 // K (bytes) per stage

}  // namespace

template <int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_f8_kernel(const uint8_t* __restrict__ A, int lda, const uint8_t* __restrict__ B, int ldb,
                    void* __restrict__ out, int ldc, int M, int N, int K, int tiles_n, int nblocks, int gm,
                    const float* __restrict__ rowscale, const float* __restrict__ colscale,
                    const RopeKvParams rp) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;
  int m0, n0;
  tile_origin(nblocks, tiles_n, gm, m0, n0);

  // DMA: wave w, instruction j fills tile rows (2w + j)*16 + lane/4, chunk
  // slot lane % 4 (holding logical chunk slot ^ ((row >> 2) & 3)).
  const int lr = lane >> 2;
  const int kc = (lane & 3) ^ ((lr >> 2) & 3);
  const uint8_t* pa[2];
  const uint8_t* pb[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ra = min(m0 + wid * 32 + j * 16 + lr, M - 1);
    const int rb = min(n0 + wid * 32 + j * 16 + lr, N - 1);
    pa[j] = A + (size_t)ra * lda + kc * 16;
    pb[j] = B + (size_t)rb * ldb + kc * 16;
  }
  const int nk = K / KS8;

  auto issue = [&](auto Sc, int st) {
    char* L = reinterpret_cast<char*>(stage_buf<decltype(Sc)::value>());
    const int k0 = st * KS8;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_global_load_lds(pa[j] + k0, L + (wid * 2 + j) * 1024, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(pb[j] + k0, L + TILE * KS8 + (wid * 2 + j) * 1024, 16, 0, 0);
    }
  };

  const int lrow = lane & 31, hl = lane >> 5;
  const int sw = (lrow >> 2) & 3;
  const int aoff = (wm * 128 + lrow) * KS8, boff = TILE * KS8 + (wn * 64 + lrow) * KS8;
  const int so0 = (hl ^ sw) * 16, so1 = ((2 + hl) ^ sw) * 16;
  i32x8 fa[2][4], fb[2][2];
  auto frag = [&](const char* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p + so0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + so1);
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  auto fread = [&](auto Sc, auto Pc) {
    constexpr int P = decltype(Pc)::value;
    const char* L = reinterpret_cast<const char*>(stage_buf<decltype(Sc)::value>());
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[P][i] = frag(L + aoff + i * 32 * KS8);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[P][j] = frag(L + boff + j * 32 * KS8);
  };
  f32x16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;
  auto mm = [&](auto Pc) {
    constexpr int P = decltype(Pc)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[P][j], fa[P][i], acc[j][i], 0, 0, 0, 127,
                                                                    0, 127);
  };

  // Prologue: stages 0..3 in flight, wait for stage 0, read it, then stage 4.
  issue(Ic<0>{}, 0);
  issue(Ic<1>{}, min(1, nk - 1));
  issue(Ic<2>{}, min(2, nk - 1));
  issue(Ic<3>{}, min(3, nk - 1));
  __builtin_amdgcn_s_waitcnt(WAIT_VM12_LGKM0);
  lds_barrier();
  fread(Ic<0>{}, Ic<0>{});
  issue(Ic<4>{}, min(4, nk - 1));

  // Stage kt (ring buffer C = kt % 5, fragments in set P = kt % 2): wait for
  // this wave's loads of stage kt + 1 and this wave's fragment reads, publish
  // stage kt + 1 with the barrier (every wave has then also read stage kt),
  // refill buffer C with stage kt + 5, read stage kt + 1, multiply stage kt.
  // Past the end the ring re-reads the last stage into buffers whose contents
  // are never multiplied, which keeps the vmcnt bookkeeping uniform.
  auto step = [&](auto Cc, auto Pc, int kt) {
    constexpr int C = decltype(Cc)::value, P = decltype(Pc)::value;
    __builtin_amdgcn_s_waitcnt(WAIT_VM12_LGKM0);
    lds_barrier();
    issue(Ic<C>{}, min(kt + 5, nk - 1));
    fread(Ic<(C + 1) % 5>{}, Ic<1 - P>{});
    mm(Ic<P>{});
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read (ring refill)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS reads
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  for (int kt = 0; kt < nk; kt += 10) {
    step(Ic<0>{}, Ic<0>{}, kt);
    if (kt + 1 >= nk) break;
    step(Ic<1>{}, Ic<1>{}, kt + 1);
    if (kt + 2 >= nk) break;
    step(Ic<2>{}, Ic<0>{}, kt + 2);
    if (kt + 3 >= nk) break;
    step(Ic<3>{}, Ic<1>{}, kt + 3);
    if (kt + 4 >= nk) break;
    step(Ic<4>{}, Ic<0>{}, kt + 4);
    if (kt + 5 >= nk) break;
    step(Ic<0>{}, Ic<1>{}, kt + 5);
    if (kt + 6 >= nk) break;
    step(Ic<1>{}, Ic<0>{}, kt + 6);
    if (kt + 7 >= nk) break;
    step(Ic<2>{}, Ic<1>{}, kt + 7);
    if (kt + 8 >= nk) break;
    step(Ic<3>{}, Ic<0>{}, kt + 8);
    if (kt + 9 >= nk) break;
    step(Ic<4>{}, Ic<1>{}, kt + 9);
  }

  __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
  lds_barrier();
  dma_epilogue<EPI>(acc, tid, m0, n0, M, N, out, ldc, colscale, rowscale, rp);
}

bool gemm_f8_ok(int epi, const void* A, int lda, const void* B, int ldb, const void* out, int ldc, int M, int N,
                int K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % KS8 != 0 || N % 8 != 0) return false;
  if (lda % 16 || ldb % 16 || ldc % 8) return false;
  const uintptr_t al = (uintptr_t)A | (uintptr_t)B | (uintptr_t)out;
  if (al & 15) return false;
  if (epi == GEPI_SWIGLU_BF16 && N % 64 != 0) return false;
  return epi == GEPI_STORE_F32 || epi == GEPI_SWIGLU_BF16 || epi == GEPI_QKV_ROPE;
}

hipError_t gemm_f8(int epi, const void* A, int lda, const void* B, int ldb, void* out, int ldc, int M, int N,
                   int K, hipStream_t s, const float* rowscale, const float* colscale, const RopeKvParams* rope) {
  if (!gemm_f8_ok(epi, A, lda, B, ldb, out, ldc, M, N, K)) return hipErrorInvalidValue;
  if (colscale != nullptr && ((uintptr_t)colscale & 15)) return hipErrorInvalidValue;
  RopeKvParams rp{};
  if (epi == GEPI_QKV_ROPE) {
    if (rope == nullptr || !gemm_dma_rope_ok(*rope, M, N)) return hipErrorInvalidValue;
    rp = *rope;
  }
  const int tn = (N + TILE - 1) / TILE, tm = (M + TILE - 1) / TILE;
  const int nb = tn * tm;
  const int gm = gemm_tile_group();
  const uint8_t* a = (const uint8_t*)A;
  const uint8_t* b = (const uint8_t*)B;
  switch (epi) {
    case GEPI_SWIGLU_BF16:
      gemm_f8_kernel<GEPI_SWIGLU_BF16><<<nb, 512, 0, s>>>(a, lda, b, ldb, out, ldc, M, N, K, tn, nb, gm, rowscale, colscale, rp);
      break;
    case GEPI_STORE_F32:
      gemm_f8_kernel<GEPI_STORE_F32><<<nb, 512, 0, s>>>(a, lda, b, ldb, out, ldc, M, N, K, tn, nb, gm, rowscale, colscale, rp);
      break;
    case GEPI_QKV_ROPE:
      gemm_f8_kernel<GEPI_QKV_ROPE><<<nb, 512, 0, s>>>(a, lda, b, ldb, out, ldc, M, N, K, tn, nb, gm, rowscale, colscale, rp);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fsk
