// Causal prefill attention for head_dim 128 (bf16 operands, fp32 softmax and
// accumulation): GQA, causal mask including the diagonal, softmax of
// q.k / sqrt(d) ("Failed Star (fs)", How it's built: grouped-query attention
// over the cache), computed flash-style so the S x S scores never leave
// registers.
//
// Work split.  A workgroup takes 128 queries of the two query heads that share
// one KV head (workgroups ordered longest first across all heads and
// sequences): 8 waves, two per SIMD; wave w owns 32 queries (one 32-column
// block) of head 2y + w/4, so the two waves on a SIMD overlap one's
// exponentials with the other's products.  Each wave reads 32 KB of K and V
// fragments from LDS per 64-key tile for 32 MFMAs, which puts the tile loop
// close to the LDS bandwidth (a 64-query wave would halve that traffic but
// needs about twice the registers, leaving one wave per SIMD, which measured
// slower).
//
// Staging.  The K and V tiles (64 keys x 128 d, 16 KB each) go from HBM
// straight into LDS with global_load_lds through a ring of four stage buffers
// (four distinct LDS objects, loop unrolled by four so each access names its
// buffer statically); tile t+3 is requested once tile t has been multiplied,
// and the wait for tile t+1 is an explicit vmcnt before the tile's barrier.
// The copies are written as inline global_load_lds instructions: the
// compiler's tracking of LDS written by DMA does not cover the transposing V
// reads, and with the builtin it put a wait for every copy in flight (tiles
// t+1 and t+2) in front of tile t's V reads.  Nothing else in the tile loop
// touches global memory, so the explicit waits below are the only ones.
// Both tiles keep the cache's row-major [key][d] layout;
// the 16-B chunk c of key row k sits at chunk slot c ^ g(k) with
// g(k) = ((k & 3) << 2) | ((k >> 2) & 3): any 16 consecutive rows see a
// permutation of the 16 slots (the K fragment reads), and 4 consecutive rows
// land their 4-chunk groups in 4 different bank quarters (the transposed V
// reads), so neither conflicts.
//
// Products.  Scores are computed transposed, S^T = K . Q^T (keys on rows, the
// lane's query on the column), so softmax max and sum are reductions over a
// lane's own registers plus one exchange with the lane 32 away.  The
// probabilities then feed O^T += V^T . P^T straight from the accumulators: in a
// 16-key step, lane half h holds keys {4h..4h+3, 8+4h..8+4h+3}; the V^T
// operand is read in the same key order with two ds_read_b64_tr_b16, which
// hand each lane 4 consecutive keys of one d column (within a 16-lane group,
// lane t receives element t % 4 of the 8-byte rows addressed by lanes
// t / 4 + 4e, e = 0..3).
//
// Softmax in base 2 with a lazily moved running max m (the output is rescaled
// only when a score exceeds it by more than 8, i.e. p > 2^8); exact either way
// since the final division uses the matching sum.  q arrives pre-multiplied
// by scale * log2(e) and every score accumulator starts at -m, so the MFMA
// returns exponents ready for exp2; when m moves, the tile in hand is shifted
// by the same amount.  FIXED: the per-head q/k RMSNorm bounds every score of
// the layer by a constant m (|q'| <= sqrt(d) max|g_q| whatever q was, the
// same for k', and RoPE keeps lengths); with m <= 63 every p = 2^s lies in
// [2^-63, 2^63], a normal fp32 and bf16 number, and the sums stay far from
// overflow, so no shift is needed at all: the score accumulators start at 0
// and the tile max, its exchange and the rescale test go away.
#include "common.h"
#include "kernels.h"

namespace fsk {

namespace {

constexpr int FD = 128;              // head_dim
constexpr int FBKV = 64;             // keys per tile
constexpr int FTILE = FBKV * FD;     // elements per K (or V) tile
constexpr float FLOG2E = 1.4426950408889634f;
constexpr float FLAZY = 8.0f;

__shared__ __attribute__((aligned(1024))) bf16 f_stage0[2 * FTILE];   // K tile, then V tile
__shared__ __attribute__((aligned(1024))) bf16 f_stage1[2 * FTILE];
__shared__ __attribute__((aligned(1024))) bf16 f_stage2[2 * FTILE];
__shared__ __attribute__((aligned(1024))) bf16 f_stage3[2 * FTILE];

template <int S> __device__ __forceinline__ bf16* fbuf() {
  return S == 0 ? f_stage0 : S == 1 ? f_stage1 : S == 2 ? f_stage2 : f_stage3;
}
template <int V> struct Fc { static constexpr int value = V; };

__device__ __forceinline__ int fswz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ float fmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// s_waitcnt immediates (vmcnt low bits [3:0] and high bits [15:14]; expcnt [6:4]; lgkmcnt [11:8])
constexpr int FWAIT_VM0 = 0xF70;
__device__ __forceinline__ void fbarrier() { asm volatile("s_barrier" ::: "memory"); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4: lane l's 16
// bytes land at lds + 16 l), written out so that the compiler does not track
// it: its tracking of LDS written by DMA does not cover the transposing LDS
// reads, before which it would otherwise wait for every copy in flight; the
// kernel's own vmcnt waits and barriers order each tile's copies.
__device__ __forceinline__ void dma16(const bf16* g, bf16* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)lds;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(la), "v"(g) : "memory", "m0");
}

__device__ __forceinline__ bf16x4 tr_read(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

}  // namespace

template <bool FIXED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_fa_kernel(const AttnPrefillParams p, const bf16* __restrict__ kcache,
                            const bf16* __restrict__ vcache, const bf16* __restrict__ qin,
                            bf16* __restrict__ out) {
  constexpr int NW = 8;              // waves per workgroup (two per SIMD)
  constexpr int WPH = NW / 2;        // waves per query head
  constexpr int DPW = 16 / NW;       // DMA instructions per wave per K (or V) tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;
  int qt, hy, b;
  longest_first(blockIdx.x, (S + 127) / 128, p.nq / 2, p.B, qt, hy, b);
  const int h = hy * 2 + wid / WPH;
  const int j = h / (p.nq / p.nkv);
  const int q0 = qt * 128;
  const int wq0 = q0 + (wid % WPH) * 32;
  const int slot = p.slots[b];
  const size_t kvoff = (size_t)slot * p.slot_stride + (size_t)j * p.head_stride;
  const bf16* kg = kcache + kvoff;
  const bf16* vg = vcache + kvoff;

  const int kend = min(q0 + 128, S);                  // keys the workgroup needs
  const int ntile = (kend + FBKV - 1) / FBKV;

  // DMA: instruction i of wave w fills key rows 4 (DPW w + i) + lane/16, chunk
  // slot lane % 16; keys past S re-read key S-1 (finite, and masked to p = 0).
  const int drow = lane >> 4, dslot = lane & 15;
  auto issue = [&](auto Cc, int t) {
    bf16* L = fbuf<decltype(Cc)::value>();
    const int k0 = t * FBKV;
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int R0 = 4 * (DPW * wid + i);
      const int R = R0 + drow;
      const int key = min(k0 + R, S - 1);
      const size_t go = (size_t)key * FD + (size_t)((dslot ^ fswz(R)) * 8);
      dma16(kg + go, L + R0 * FD);
      dma16(vg + go, L + FTILE + R0 * FD);
    }
  };

  // the lane's query as the B operand of S^T (d = 16 ks + 8 half + e)
  bf16x8 qf[FD / 16];
  {
    const int q = min(wq0 + col, S - 1);
    const bf16* qrow = qin + ((size_t)b * S + q) * p.nq * FD + (size_t)h * FD;
#pragma unroll
    for (int ks = 0; ks < FD / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + half * 8);
  }

  // per-lane fragment addressing
  const int swk = fswz(col);                                   // K rows kb*32 + col
  const int vr = 4 * half + ((lane & 15) >> 2);                // V key row (mod 16) of the first transposed read
  const int swv1 = fswz(vr), swv2 = fswz(vr + 8);
  const int vcb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);   // chunk within a 32-d block
  const int vh = (lane & 1) * 4;                               // element offset of the 8-byte half
  const int qme = min(wq0 + col, S - 1);                       // the lane's query (clamped)

  float m_run = 0.f, l_run = 0.f;   // running max: set from the first tile's max (FIXED: stays 0)
  f32x16 o[4];   // O^T blocks [d block]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  f32x16 sc[2][2];   // scores of two tiles in flight: [tile parity][key block]
  bf16x8 pb[4];      // probabilities of the current tile, one per 16-key step

  // S^T of the tile in buffer C (keys on rows, the lane's query on the column)
  auto scores = [&](auto Cc, f32x16* sd) {
    const bf16* LK = fbuf<decltype(Cc)::value>();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sd[kb][r] = FIXED ? 0.f : -m_run;
#pragma unroll
    for (int ks = 0; ks < FD / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(LK + (kb * 32 + col) * FD + (((2 * ks + half) ^ swk) << 3));
        sd[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sd[kb], 0, 0, 0);
      }
  };
  // causal / ragged mask, tile max, lazy move of the running max
  auto mask_max = [&](f32x16* sv, int t) {
    const int k0 = t * FBKV;
    if (k0 + FBKV - 1 > wq0 || k0 + FBKV > S) {
      const int lim = qme - k0 - half * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + (r >> 2) * 8 + (r & 3) > lim) sv[kb][r] = -INFINITY;
    }
    if constexpr (FIXED) return 0.f;   // FIXED: masking only, done as a tile turns into probabilities
    // two independent max3 chains over the 32 scores
    float ma = fmax3(sv[0][0], sv[0][1], sv[0][2]), mb = fmax3(sv[1][0], sv[1][1], sv[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      ma = fmax3(ma, sv[0][r], sv[0][r + 1]);
      mb = fmax3(mb, sv[1][r], sv[1][r + 1]);
    }
    const float mt = fmax3(ma, mb, fmaxf(sv[0][15], sv[1][15]));
    return pair32_max(mt);   // relative to m_run
  };
  // move m_run when the tile's max (relative to it) exceeds FLAZY, or always
  // for the first tile; the unexponentiated tile sv follows the move
  auto rescale = [&](float mt, f32x16* sv, bool first) {
    if constexpr (FIXED) return;
    if (first || mt > FLAZY) {
      const float corr = __builtin_amdgcn_exp2f(-mt);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= corr;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[kb][r] -= mt;
      m_run += mt;
    }
  };
  // p = 2^(s - m), row sum, bf16 operands for the 16-key steps
  auto probs = [&](f32x16* sv, int t) {
    if constexpr (FIXED) mask_max(sv, t);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(sv[kb][r]);
        ls += e;
        pb[kb * 2 + (r >> 3)][r & 7] = (bf16)e;
      }
    l_run += pair32_sum(ls);
  };
  // O^T += V^T . P^T over the tile in buffer C
  auto pv = [&](auto Cc) {
    const bf16* LV = fbuf<decltype(Cc)::value>() + FTILE;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int kb = st >> 1, s2 = st & 1;
      const bf16* v1 = LV + (kb * 32 + 16 * s2 + vr) * FD + vh;
      const bf16* v2 = v1 + 8 * FD;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int c = (db << 2) | vcb;
        const bf16x4 lo = tr_read(v1 + ((c ^ swv1) << 3));
        const bf16x4 hi = tr_read(v2 + ((c ^ swv2) << 3));
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[st], o[db], 0, 0, 0);
      }
    }
  };

  // vmcnt immediates: this wave issues 2 * DPW loads per tile
  constexpr int W1 = (2 * DPW) | 0x70;        // one later tile may stay outstanding
  constexpr int W2 = (4 * DPW) | 0x70;        // two later tiles may stay outstanding
  issue(Fc<0>{}, 0);
  issue(Fc<1>{}, min(1, ntile - 1));
  issue(Fc<2>{}, min(2, ntile - 1));
  __builtin_amdgcn_s_waitcnt(W2);             // tile 0 landed
  fbarrier();
  scores(Fc<0>{}, sc[0]);
  if constexpr (!FIXED) rescale(mask_max(sc[0], 0), sc[0], true);
  __builtin_amdgcn_s_waitcnt(W1);             // tile 1 landed
  fbarrier();

  // Iteration t (tile t in buffer C): the scores of tile t+1 go to the matrix
  // unit while the vector unit turns tile t's scores into probabilities; then
  // tile t's P.V products run while tile t+1 is masked and its max taken.
  // Tile t+3 is requested into the buffer tile t-1 left, and tile t+2 must
  // have landed before the barrier that ends the iteration.  Past the last
  // tile the ring holds re-reads of it, whose scores are fully masked.
  auto iter = [&](auto Cc, int t) {
    constexpr int C = decltype(Cc)::value;
    f32x16* cur = sc[C & 1];
    f32x16* nxt = sc[(C + 1) & 1];
    scores(Fc<(C + 1) & 3>{}, nxt);
    probs(cur, t);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
    }
    const float mt = FIXED ? 0.f : mask_max(nxt, t + 1);
    pv(Cc);
    rescale(mt, nxt, false);
    issue(Fc<(C + 3) & 3>{}, min(t + 3, ntile - 1));
    __builtin_amdgcn_s_waitcnt(W1);
    fbarrier();
  };
  for (int t = 0; t < ntile; t += 4) {
    iter(Fc<0>{}, t);
    if (t + 1 < ntile) iter(Fc<1>{}, t + 1);
    if (t + 2 < ntile) iter(Fc<2>{}, t + 2);
    if (t + 3 < ntile) iter(Fc<3>{}, t + 3);
  }
  __builtin_amdgcn_s_waitcnt(FWAIT_VM0);   // no LDS DMA may outlive the workgroup

  // O^T[d][q] / l -> out[(b*S + q), h*D + d]
  const int q = wq0 + col;
  if (q < S) {
    const float inv = 1.f / l_run;
    bf16* orow = out + ((size_t)b * S + q) * p.nq * FD + (size_t)h * FD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[db][g * 4 + i] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + g * 8 + half * 4) = v;
      }
  }
}

bool attn_prefill_fa_ok(const AttnPrefillParams& p) {
  return p.d == FD && p.q_dt == DT_BF16 && p.kv_dt == DT_BF16 && p.o_dt == DT_BF16 &&
         p.nkv > 0 && p.nq % p.nkv == 0 && (p.nq / p.nkv) % 2 == 0;
}

hipError_t attn_prefill_fa(const AttnPrefillParams& p, hipStream_t s) {
  if (std::fabs(p.q_prescale - p.scale * FLOG2E) > 1e-6f * p.scale * FLOG2E) return hipErrorInvalidValue;
  const int grid = (p.S + 127) / 128 * (p.nq / 2) * p.B;
  if (p.m_fixed > 0.f && p.m_fixed <= ATTN_FIXED_SHIFT_MAX)
    attn_prefill_fa_kernel<true><<<grid, 512, 0, s>>>(p, (const bf16*)p.kcache, (const bf16*)p.vcache,
                                                       (const bf16*)p.q, (bf16*)p.out);
  else
    attn_prefill_fa_kernel<false><<<grid, 512, 0, s>>>(p, (const bf16*)p.kcache, (const bf16*)p.vcache,
                                                        (const bf16*)p.q, (bf16*)p.out);
  return hipGetLastError();
}

}  // namespace fsk
