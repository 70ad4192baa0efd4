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
// unrolled by five, so every access names its buffer statically; the
// compiler's tracking of LDS DMA then needs no blanket vmcnt(0) before each
// fragment read, and the one wait per stage is the explicit vmcnt(12) (this
// wave's four loads for stage k+1 done) before the stage's single barrier.
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
#include "common.h"
#include "kernels.h"

namespace fsk {

namespace {

constexpr int DK = 32;                  // K per stage
constexpr int TILE = 256;               // output tile edge
constexpr int STAGE = 2 * TILE * DK;    // bf16 elements per stage: A rows then B rows (32 KB)

__shared__ __attribute__((aligned(1024))) bf16 g_stage0[STAGE];
__shared__ __attribute__((aligned(1024))) bf16 g_stage1[STAGE];
__shared__ __attribute__((aligned(1024))) bf16 g_stage2[STAGE];
__shared__ __attribute__((aligned(1024))) bf16 g_stage3[STAGE];
__shared__ __attribute__((aligned(1024))) bf16 g_stage4[STAGE];

template <int S> __device__ __forceinline__ bf16* stage_buf() {
  return S == 0 ? g_stage0 : S == 1 ? g_stage1 : S == 2 ? g_stage2 : S == 3 ? g_stage3 : g_stage4;
}
// stage buffer w (0..3) as raw bytes
__device__ __forceinline__ char* stage_bytes(int w) {
  return reinterpret_cast<char*>(w == 0 ? g_stage0 : w == 1 ? g_stage1 : w == 2 ? g_stage2 : g_stage3);
}
// 16 KB of LDS for wave w's epilogue: half (w & 1) of stage buffer w >> 1
__device__ __forceinline__ char* wave_region(int w) {
  char* b = reinterpret_cast<char*>((w >> 1) == 0 ? g_stage0 : (w >> 1) == 1 ? g_stage1 : (w >> 1) == 2 ? g_stage2 : g_stage3);
  return b + (w & 1) * 16384;
}

template <int V> struct Ic { static constexpr int value = V; };

// s_waitcnt immediates (gfx9 encoding: vmcnt low bits [3:0], high bits [15:14];
// expcnt [6:4]; lgkmcnt [11:8]).
constexpr int WAIT_VM12_LGKM0 = 0x7C;               // vmcnt(12) lgkmcnt(0)
constexpr int WAIT_VM0_LGKM0 = 0x70;                // vmcnt(0) lgkmcnt(0)

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace

// QKV epilogue of a prefill: the tile's 256 tokens x 256 columns are two
// heads of 128 (all q, all k or all v: the section boundaries fall on tile
// boundaries).  The fp32 products are staged in LDS 128 tokens at a time (the
// four waves of one token half each write their 128 x 64 block, 32 KB, into
// one stage buffer); then per (token, head) the q/k heads get the per-head
// RMSNorm and rotate-half RoPE over all 128 dims (q also the attention's
// pre-scale) and go to the q buffer or the K cache, and v goes to the V cache
// as it is.  The arithmetic is the standalone norm/RoPE pass's, step for step,
// on the same fp32 inputs, so the results are the same bits.  Eight lanes per
// (token, head): lane `sub` holds dims [8 sub, 8 sub + 8) (block of wave
// 2 head) and their partners [64 + 8 sub, ...) (block of wave 2 head + 1).
// Row m of a staged block is 64 floats in 16 chunks of 16 B, chunk c at slot
// c ^ (m & 15).
__device__ __forceinline__ void qkv_rope_epilogue(const RopeKvParams& p, const f32x16 (&acc)[2][4], int m0,
                                                  int n0, int M, int tid) {
  constexpr int D = 128;
  const int lane = tid & 63, wid = tid >> 6, wm = wid >> 2, wn = wid & 3;
  const int lrow = lane & 31, hl = lane >> 5;
  const int hsec = n0 / D;                         // first of the tile's two heads in q|k|v order
  const bool is_q = hsec < p.nq, is_k = !is_q && hsec < p.nq + p.nkv;
  const int sub = tid & 7;
  const float* g = is_q ? p.gq : p.gk;
  float g0[8], g1[8];
  load8(g + 8 * sub, g0);
  load8(g + 64 + 8 * sub, g1);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
      char* R = stage_bytes(wn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = i * 32 + lrow;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[j][i][4 * gq + e];
            const int cc = j * 8 + 2 * gq + hl;
            *reinterpret_cast<f32x4*>(R + m * 256 + ((cc ^ (m & 15)) << 4)) = v;
          }
      }
    }
    lds_barrier();
#pragma unroll 2
    for (int it = 0; it < 4; ++it) {
      const int item = it * 512 + tid;
      const int hd = (item >> 3) & 1, mr = item >> 4;      // head of the tile, row of the half
      const int row = half * 128 + mr;
      const char* RA = stage_bytes(2 * hd) + mr * 256;
      const char* RB = stage_bytes(2 * hd + 1) + mr * 256;
      float x0[8], x1[8];
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(RA + (((2 * sub) ^ (mr & 15)) << 4));
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(RA + (((2 * sub + 1) ^ (mr & 15)) << 4));
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(RB + (((2 * sub) ^ (mr & 15)) << 4));
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(RB + (((2 * sub + 1) ^ (mr & 15)) << 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) { x0[e] = a0[e]; x0[4 + e] = a1[e]; x1[e] = b0[e]; x1[4 + e] = b1[e]; }
      const int t = min(m0 + row, M - 1);
      const int b = t / p.S_per, pos = t % p.S_per;
      const int hh = hsec + hd;
      if (is_q || is_k) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x0[e], x0[e], fmaf(x1[e], x1[e], ss));
        ss = group_sum<8>(ss);
        const float inv = rsqrtf(__fadd_rn(ss / (float)D, p.eps));
        float cs[8], sn[8];
        load8(p.cos_t + (size_t)pos * (D / 2) + 8 * sub, cs);
        load8(p.sin_t + (size_t)pos * (D / 2) + 8 * sub, sn);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = x0[e] * inv * g0[e], c = x1[e] * inv * g1[e];
          const float y0 = fmaf(a, cs[e], -(c * sn[e])), y1 = fmaf(c, cs[e], a * sn[e]);
          x0[e] = is_q ? y0 * p.qscale : y0;
          x1[e] = is_q ? y1 * p.qscale : y1;
        }
      }
      if (m0 + row < M) {
        bf16* dst;
        if (is_q) {
          dst = reinterpret_cast<bf16*>(p.qout) + (size_t)t * p.nq * D + (size_t)hh * D;
        } else {
          const int j = is_k ? hh - p.nq : hh - p.nq - p.nkv;
          const size_t o = (size_t)p.slots[b] * p.slot_stride + (size_t)j * p.head_stride + (size_t)pos * D;
          dst = reinterpret_cast<bf16*>(is_k ? p.kcache : p.vcache) + o;
        }
        u32x4 u0, u1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u0[i] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x0[2 * i]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)x0[2 * i + 1]) << 16);
          u1[i] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x1[2 * i]) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)x1[2 * i + 1]) << 16);
        }
        *reinterpret_cast<u32x4*>(dst + 8 * sub) = u0;
        *reinterpret_cast<u32x4*>(dst + 64 + 8 * sub) = u1;
      }
    }
    lds_barrier();                                 // the next half reuses the buffers
  }
}

template <int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_dma_kernel(const bf16* __restrict__ A, int lda, const bf16* __restrict__ A_lo,
                  const bf16* __restrict__ B, int ldb, void* __restrict__ out, int ldc,
                  int M, int N, int K, int tiles_n, int nblocks, const float* __restrict__ colscale,
                  const RopeKvParams rp) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;
  // XCD-aware renumbering: the hardware deals workgroups round-robin over the
  // 8 XCDs; consecutive tiles (sharing A rows / B rows) go to one XCD's L2.
  int bid = blockIdx.x;
  if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
  const int n0 = (bid % tiles_n) * TILE, m0 = (bid / tiles_n) * TILE;

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

  auto issue = [&](auto Sc, int st) {
    bf16* L = stage_buf<decltype(Sc)::value>();
    const bool lo = st >= nk0;
    const int k0 = (lo ? st - nk0 : st) * DK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_global_load_lds((lo ? pl[j] : pa[j]) + k0, L + (wid * 2 + j) * 16 * DK, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(pb[j] + k0, L + TILE * DK + (wid * 2 + j) * 16 * DK, 16, 0, 0);
    }
  };

  const int lrow = lane & 31;
  const int sw = (lrow >> 2) & 3;
  const int aoff = (wm * 128 + lrow) * DK, boff = TILE * DK + (wn * 64 + lrow) * DK;
  const int so0 = ((lane >> 5) ^ sw) * 8, so1 = ((2 + (lane >> 5)) ^ sw) * 8;
  bf16x8 fa[2][4], fb[2][2];
  auto fread = [&](auto Sc, int set, int q) {
    const bf16* L = stage_buf<decltype(Sc)::value>();
    const int so = q ? so1 : so0;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[set][i] = *reinterpret_cast<const bf16x8*>(L + aoff + i * 32 * DK + so);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[set][j] = *reinterpret_cast<const bf16x8*>(L + boff + j * 32 * DK + so);
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
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[set][j], fa[set][i], acc[j][i], 0, 0, 0);
  };

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

  // ---- epilogue: drain the ring, then each wave stages its 128x64 block in
  // its own 16 KB of LDS and writes whole rows.
  __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGKM0);
  lds_barrier();
  char* R = wave_region(wid);
  const int hl = lane >> 5;
  const int mrow0 = m0 + wm * 128;
  const int ncol0 = n0 + wn * 64;
  if (colscale != nullptr) {
    // per-column scale; columns past N (clamped reads) are never stored
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

  if constexpr (EPI == GEPI_QKV_ROPE) {
    qkv_rope_epilogue(rp, acc, m0, n0, M, tid);
    return;
  }
  if (EPI == GEPI_STORE_BF16) {
    // 128 rows x 128 B; chunk c of row m at slot c ^ (m & 7)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = i * 32 + lrow;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (bf16)acc[j][i][4 * g + e];
          const int c = j * 4 + g;
          *reinterpret_cast<bf16x4*>(R + m * 128 + ((c ^ (m & 7)) << 4) + hl * 8) = v;
        }
    }
    bf16* o = reinterpret_cast<bf16*>(out);
    const int c = lane & 7;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int m = it * 8 + (lane >> 3);
      const u32x4 v = *reinterpret_cast<const u32x4*>(R + m * 128 + ((c ^ (m & 7)) << 4));
      const int gm = mrow0 + m, gn = ncol0 + c * 8;
      if (gm < M && gn < N) *reinterpret_cast<u32x4*>(o + (size_t)gm * ldc + gn) = v;
    }
  } else if (EPI == GEPI_SWIGLU_BF16) {
    // the wave's 64 packed columns are one [32 gate | 32 up] pair -> 32 outputs;
    // 128 rows x 64 B, chunk c of row m at slot c ^ (m & 3)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = i * 32 + lrow;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(silu(acc[0][i][4 * g + e]) * acc[1][i][4 * g + e]);
        *reinterpret_cast<bf16x4*>(R + m * 64 + ((g ^ (m & 3)) << 4) + hl * 8) = v;
      }
    }
    bf16* o = reinterpret_cast<bf16*>(out);
    const int c = lane & 3;
    const int f0 = ncol0 / 2, nf = N / 2;
#pragma unroll 4
    for (int it = 0; it < 8; ++it) {
      const int m = it * 16 + (lane >> 2);
      const u32x4 v = *reinterpret_cast<const u32x4*>(R + m * 64 + ((c ^ (m & 3)) << 4));
      const int gm = mrow0 + m, f = f0 + c * 8;
      if (gm < M && f < nf) *reinterpret_cast<u32x4*>(o + (size_t)gm * ldc + f) = v;
    }
  } else {
    // fp32: two passes of 64 rows x 256 B; chunk cc of row m at slot cc ^ (m & 15)
    float* o = reinterpret_cast<float*>(out);
    const int c = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * h + ii;
        const int m = ii * 32 + lrow;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[j][i][4 * g + e];
            const int cc = j * 8 + 2 * g + hl;
            *reinterpret_cast<f32x4*>(R + m * 256 + ((cc ^ (m & 15)) << 4)) = v;
          }
      }
      const int gn = ncol0 + c * 4, gnc = min(gn, N - 4);
      for (int it0 = 0; it0 < 16; it0 += 4) {
        f32x4 old[4];
        if (EPI == GEPI_RESID_F32) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int gmc = min(mrow0 + h * 64 + (it0 + u) * 4 + (lane >> 4), M - 1);
            old[u] = *reinterpret_cast<const f32x4*>(o + (size_t)gmc * ldc + gnc);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int m = (it0 + u) * 4 + (lane >> 4);
          f32x4 v = *reinterpret_cast<const f32x4*>(R + m * 256 + ((c ^ (m & 15)) << 4));
          const int gm = mrow0 + h * 64 + m;
          if (EPI == GEPI_RESID_F32) v += old[u];
          if (gm < M && gn < N) *reinterpret_cast<f32x4*>(o + (size_t)gm * ldc + gn) = v;
        }
      }
    }
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
                    const RopeKvParams* rope) {
  if (colscale != nullptr && ((uintptr_t)colscale & 15)) return hipErrorInvalidValue;
  RopeKvParams rp{};
  if (epi == GEPI_QKV_ROPE) {
    if (rope == nullptr || !gemm_dma_rope_ok(*rope, M, N)) return hipErrorInvalidValue;
    rp = *rope;
  }
  const int tn = (N + TILE - 1) / TILE, tm = (M + TILE - 1) / TILE;
  const int nb = tn * tm;
  const bf16* a = (const bf16*)A;
  const bf16* b = (const bf16*)B;
  const bf16* al = (const bf16*)A_lo;
  switch (epi) {
    case GEPI_STORE_BF16:
      gemm_dma_kernel<GEPI_STORE_BF16><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, colscale, rp);
      break;
    case GEPI_RESID_F32:
      gemm_dma_kernel<GEPI_RESID_F32><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, colscale, rp);
      break;
    case GEPI_SWIGLU_BF16:
      gemm_dma_kernel<GEPI_SWIGLU_BF16><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, colscale, rp);
      break;
    case GEPI_STORE_F32:
      gemm_dma_kernel<GEPI_STORE_F32><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, colscale, rp);
      break;
    case GEPI_QKV_ROPE:
      gemm_dma_kernel<GEPI_QKV_ROPE><<<nb, 512, 0, s>>>(a, lda, al, b, ldb, out, ldc, M, N, K, tn, nb, colscale, rp);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fsk
