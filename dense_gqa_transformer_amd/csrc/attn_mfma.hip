// Causal prefill attention on MFMA (bf16 operands, fp32 softmax and accumulation).
//
// Same mathematics as the vector path (GQA, causal mask including the
// diagonal, softmax of q.k/sqrt(d)); flash-style tiling so the S x S score
// matrix never leaves registers.
//
// One workgroup = HPW query heads of one KV group x 128 queries, 4 waves per
// head; each wave owns 32 queries (head_dim 64 / 128: two heads when the group
// has an even count; head_dim 256: one, its output accumulators take 128
// registers per lane).  The heads of a group share every
// key/value tile, staged once in LDS: K row-major [key][d], V transposed
// [d][key].  The next tile is fetched into registers while the current one is
// being used.  Each wave computes the transposed scores S^T = K . Q^T (keys on
// rows, its 32 queries on columns) with v_mfma_f32_32x32x16_bf16, so every
// lane owns one query column: the softmax max / sum is a reduction over the
// lane's own registers plus one exchange with the lane 32 away.  The
// probabilities then feed O^T += V^T . P^T straight from the accumulator
// registers: for a 16-key step, lane half h holds keys {4h..4h+3,
// 8+4h..8+4h+3} in its registers, and the V^T fragment is read in the same
// key order, so A and B agree on k whatever order the unit reduces in.
//
// Softmax in base 2 with a lazily updated running max: the reference max only
// moves when a score exceeds it by more than 2^8, so the rescale of the
// output accumulators is almost never executed; the result is exact either
// way since the final division uses the matching sum.
#include "common.h"
#include "kernels.h"

namespace fsk {

static constexpr float LOG2E_M = 1.4426950408889634f;
static constexpr float LAZY_MAX = 8.0f;   // log2 of the largest un-rescaled p

template <int D, int HPW>
__global__ __launch_bounds__(256 * HPW) void attn_prefill_mfma_kernel(const AttnPrefillParams p) {
  constexpr int BQ = 128, BKV = 64;
  constexpr int NT = 256 * HPW;     // threads
  constexpr int LDK = D + 8;        // K tile row stride (elements)
  constexpr int LDV = BKV + 4;      // V^T tile row stride (elements): 136 B, 8-byte aligned, spreads rows over banks
  constexpr int KS = D / 16;        // k-steps of the score product
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  constexpr int CH = BKV * D / 8;   // 16-byte chunks per K (or V) tile
  constexpr int CPT = CH / NT;      // chunks per thread
  constexpr int VP = (BKV / 2) * (D / 8);   // V key-pair chunks per tile
  constexpr int VPT = (VP + NT - 1) / NT;   // per thread
  static_assert(CPT >= 1 && CH % NT == 0, "tile / thread mismatch");
  __shared__ __attribute__((aligned(16))) bf16 Ks[BKV * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;
  int qt, hy, b;                                          // longest tiles first
  longest_first(blockIdx.x, (S + BQ - 1) / BQ, p.nq / HPW, p.B, qt, hy, b);
  const int h = hy * HPW + (wid >> 2);                    // this wave's query head
  const int j = h / (p.nq / p.nkv);
  const int q0 = qt * BQ;
  const int wq0 = q0 + (wid & 3) * 32;
  const int myq = wq0 + col;
  const int slot = p.slots[b];
  const size_t kvoff = (size_t)slot * p.slot_stride + (size_t)j * p.head_stride;
  const bf16* __restrict__ kg = reinterpret_cast<const bf16*>(p.kcache) + kvoff;
  const bf16* __restrict__ vg = reinterpret_cast<const bf16*>(p.vcache) + kvoff;
  const bf16* __restrict__ qg = reinterpret_cast<const bf16*>(p.q);

  // this lane's query, as the B operand of S^T = K . Q^T (d = 16*ks + 8*half + e)
  bf16x8 qf[KS];
  {
    const int qq = min(myq, S - 1);
    const bf16* qrow = qg + ((size_t)b * S + qq) * p.nq * D + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16 + half * 8);
  }
  const float c2 = p.scale * LOG2E_M;   // raw score -> base-2 exponent
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  // register staging of one K/V tile: K chunks row-major (coalesced); V as
  // pairs of consecutive keys per lane (same 8 columns), so the transposed
  // LDS writes are dwords and one instruction covers 32 consecutive dwords
  u32x4 rk[CPT];
  u32x4 rv[VPT][2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int id = tid + NT * i;
      const int kk = id / (D / 8), kc = (id % (D / 8)) * 8;
      rk[i] = (k0 + kk < S) ? *reinterpret_cast<const u32x4*>(kg + (size_t)(k0 + kk) * D + kc)
                            : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int id = min(tid + NT * i, VP - 1);            // BKV/2 key pairs x D/8 column chunks
      const int vk = (id % (BKV / 2)) * 2, vc = (id / (BKV / 2)) * 8;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        rv[i][t] = (k0 + vk + t < S) ? *reinterpret_cast<const u32x4*>(vg + (size_t)(k0 + vk + t) * D + vc)
                                     : u32x4{0, 0, 0, 0};
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int id = tid + NT * i;
      const int kk = id / (D / 8), kc = (id % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ks[kk * LDK + kc]) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int id = tid + NT * i;
      if (id >= VP) break;
      const int vk = (id % (BKV / 2)) * 2, vc = (id / (BKV / 2)) * 8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {                        // columns vc + 2q and vc + 2q + 1
        const uint32_t a = rv[i][0][q], b = rv[i][1][q];
        *reinterpret_cast<uint32_t*>(&Vt[(vc + 2 * q) * LDV + vk]) = (a & 0xffffu) | (b << 16);
        *reinterpret_cast<uint32_t*>(&Vt[(vc + 2 * q + 1) * LDV + vk]) = (a >> 16) | (b & 0xffff0000u);
      }
    }
  };

  const int kend = min(q0 + BQ, S);
  fetch(0);
  for (int k0 = 0; k0 < kend; k0 += BKV) {
    __syncthreads();                          // every wave is done with the previous tile
    stash();
    __syncthreads();
    if (k0 + BKV < kend) fetch(k0 + BKV);     // next tile in flight during this one
    if (k0 > wq0 + 31) continue;              // every query of this wave precedes the tile

    // ---- S^T for keys k0 + 32*kb + (8*(r/4) + 4*half + r%4), query myq
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {                  // two independent accumulator chains
      bf16x8 a[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        a[kb] = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + col) * LDK + ks * 16 + half * 8]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], qf[ks], s[kb], 0, 0, 0);
    }
    // ---- causal mask (only on tiles that reach past this wave's first query):
    //      key offset within the tile is a per-register constant
    if (k0 + BKV - 1 > wq0) {
      const int lim = min(myq, S - 1) - k0 - half * 4;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + (r >> 2) * 8 + (r & 3) > lim) s[kb][r] = -INFINITY;
    }
    // ---- tile max (raw units), lazily moved running max (base-2 units)
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mt = fmaxf(mt, fmaxf(s[kb][r], s[kb][r + 1]));
    mt = pair32_max(mt) * c2;
    if (mt > m_run + LAZY_MAX) {             // rare after the first tile
      const float corr = __builtin_amdgcn_exp2f(m_run - mt);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= corr;
      m_run = mt;
    }
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -m_run));
        s[kb][r] = e;
        ls += e;
      }
    l_run += pair32_sum(ls);

    // ---- O^T += V^T . P^T over four 16-key steps
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const int kb = ks2 >> 1, r0 = (ks2 & 1) * 8;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = (bf16)s[kb][r0 + e];
      const int kofs = kb * 32 + (ks2 & 1) * 16 + half * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16* vr = &Vt[(db * 32 + col) * LDV + kofs];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + 8);
        bf16x8 a;
        a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
        a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
      }
    }
  }

  // ---- O^T[d][myq] / l -> out[(b*S + myq), h*D + d]
  if (myq < S) {
    const float inv = 1.f / l_run;
    bf16* orow = reinterpret_cast<bf16*>(p.out) + ((size_t)b * S + myq) * p.nq * D + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[db][g * 4 + i] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + g * 8 + half * 4) = v;
      }
  }
}

template <int D>
static hipError_t launch_mfma(const AttnPrefillParams& p, hipStream_t s) {
  const int rep = p.nq / p.nkv;
  if constexpr (D <= 128) {
    if (rep % 2 == 0) {
      const int grid = (p.S + 127) / 128 * (p.nq / 2) * p.B;
      attn_prefill_mfma_kernel<D, 2><<<grid, 512, 0, s>>>(p);
      return hipGetLastError();
    }
  }
  {
    const int grid = (p.S + 127) / 128 * p.nq * p.B;
    attn_prefill_mfma_kernel<D, 1><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

hipError_t attn_prefill(const AttnPrefillParams& p, hipStream_t s) {
  if (p.B <= 0 || p.S <= 0) return hipSuccess;
  const bool bf = p.q_dt == DT_BF16 && p.kv_dt == DT_BF16 && p.o_dt == DT_BF16;
  if (!bf || (p.d != 128 && p.d != 64 && p.d != 256)) return attn_prefill_vec(p, s);
  if (p.d == 256) return launch_mfma<256>(p, s);    // one head per workgroup (register budget)
  return p.d == 128 ? launch_mfma<128>(p, s) : launch_mfma<64>(p, s);
}

}  // namespace fsk
