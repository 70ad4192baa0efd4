// Pieces shared by the large MFMA GEMMs (bf16 operands in gemm_dma.hip, fp8
// operands in gemm_f8.hip): the five-stage LDS ring, the wait / barrier
// helpers, and the epilogues.  Both kernels tile the output 256x256 per
// workgroup of 8 waves (2 x 4, 128x64 per wave = 4 x 2 blocks of 32x32), and
// lane l of block (i, j) holds activation row i*32 + (l % 32) and output
// columns 32 j + 8 (r / 4) + 4 (l / 32) + (r % 4) in accumulator registers r,
// whatever the operand type; a stage row is 64 B either way (32 bf16 or 64
// fp8 values).
#pragma once
#include <cstdlib>

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

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4: lane l's 16
// bytes land at lds + 16 l; lds is the same for the whole wave), written out so
// that the compiler does not track it.  Its tracking of DMA-written LDS cannot
// tell the ring's stage buffers apart and put a wait for every copy in flight
// (vmcnt(0)) in front of fragment reads of other stages, once per unrolled
// pass of the K loop.  The kernel's own vmcnt waits and barriers order every
// stage's copies; the compiler's waits for its own loads stay correct, since
// loads complete in order and untracked copies only make them wait longer.
// (The fp8 GEMM keeps the builtin: there the written-out form cost registers
// and measured slower.)
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(la), "v"(g) : "memory", "m0");
}

// Output tile of this workgroup.  The hardware deals workgroups to the 8 XCDs
// round robin; renumbering gives each XCD a contiguous range of tiles, whose
// shared operand rows its L2 then serves.  Within the range the tiles go gm
// tile rows at a time across the columns, so the 32 tiles an XCD runs at once
// cover gm rows x 32/gm columns (each activation block read by 32/gm of them,
// each weight block by gm) instead of one or two tile rows across all
// columns.  gm <= 1, or a tile-row count that gm does not divide, keeps
// row-major order.
__device__ __forceinline__ void tile_origin(int nblocks, int tiles_n, int gm, int& m0, int& n0) {
  int bid = blockIdx.x;
  if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
  const int tiles_m = nblocks / tiles_n;
  int mt, nt;
  if (gm > 1 && tiles_m % gm == 0) {
    const int per = gm * tiles_n;
    const int g = bid / per, r = bid - g * per;
    mt = g * gm + r % gm;
    nt = r / gm;
  } else {
    mt = bid / tiles_n;
    nt = bid % tiles_n;
  }
  m0 = mt * TILE;
  n0 = nt * TILE;
}

// Tile-row group of the launches (FS_GEMM_TILE_GROUP, read once; default 2:
// measured on the 4 x 4096 prefill, groups of 4 halve the fetched bytes of
// the Q/K/V and gate/up GEMMs against row-major order but run no faster, and
// groups of 2 run 2-8% faster than either).
inline int gemm_tile_group() {
  static const int g = [] {
    const char* e = std::getenv("FS_GEMM_TILE_GROUP");
    const int v = e != nullptr ? std::atoi(e) : 2;
    return (v >= 0 && v <= 16) ? v : 2;
  }();
  return g;
}


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

// Epilogue after the K loop has drained (the ring's LDS is free): optional
// per-column (weight row) and per-row (activation row) scales, then the
// store form EPI.  Columns / rows past N / M are computed on clamped reads and
// never stored.
template <int EPI>
__device__ __forceinline__ void dma_epilogue(f32x16 (&acc)[2][4], int tid, int m0, int n0, int M, int N,
                                             void* __restrict__ out, int ldc, const float* __restrict__ colscale,
                                             const float* __restrict__ rowscale, const RopeKvParams& rp) {
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;
  const int lrow = lane & 31;
  char* R = wave_region(wid);
  const int hl = lane >> 5;
  const int mrow0 = m0 + wm * 128;
  const int ncol0 = n0 + wn * 64;
  if (rowscale != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sa = rowscale[min(mrow0 + i * 32 + lrow, M - 1)];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] *= sa;
    }
  }
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
    // 128 rows x 64 B, chunk c of row m at slot c ^ ((m >> 2) & 3): a row's 64 B
    // fill one quarter of the banks (m & 3 picks it), so the 8 rows of a write
    // that share a quarter spread over its 4 chunk slots (2 per slot, the
    // minimum) instead of all landing on one
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = i * 32 + lrow;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(silu(acc[0][i][4 * g + e]) * acc[1][i][4 * g + e]);
        *reinterpret_cast<bf16x4*>(R + m * 64 + ((g ^ ((m >> 2) & 3)) << 4) + hl * 8) = v;
      }
    }
    bf16* o = reinterpret_cast<bf16*>(out);
    const int c = lane & 3;
    const int f0 = ncol0 / 2, nf = N / 2;
#pragma unroll 4
    for (int it = 0; it < 8; ++it) {
      const int m = it * 16 + (lane >> 2);
      const u32x4 v = *reinterpret_cast<const u32x4*>(R + m * 64 + ((c ^ ((m >> 2) & 3)) << 4));
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

}  // namespace
}  // namespace fsk
