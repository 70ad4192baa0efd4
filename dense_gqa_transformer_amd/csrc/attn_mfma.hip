// Causal prefill attention on MFMA (bf16 operands, fp32 softmax and accumulation).
//
// Same mathematics as the vector path (GQA, causal mask including the
// diagonal, softmax of q.k/sqrt(d)); flash-style tiling so the S x S score
// matrix never leaves registers.
//
// One workgroup = 4 waves = 128 queries of one query head; each wave owns 32
// queries.  Key/value tiles of 64 positions are staged in LDS: K row-major
// [key][d], V transposed [d][key].  Each wave computes the transposed scores
// S^T = K . Q^T (keys on rows, its 32 queries on columns) with
// v_mfma_f32_32x32x16_bf16, so every lane owns one query column: the row
// max / sum of the online softmax is a reduction over the lane's own
// registers plus one exchange with the lane 32 away.  The probabilities then
// feed O^T += V^T . P^T straight from the accumulator registers: for a
// 16-key step, lane half h holds keys {4h..4h+3, 8+4h..8+4h+3} in its
// registers, and the V^T fragment is read with the same key order, so A and
// B agree on k whatever order the unit reduces in.
#include "common.h"
#include "kernels.h"

namespace fsk {

static constexpr float LOG2E_M = 1.4426950408889634f;

template <int D>
__global__ __launch_bounds__(256) void attn_prefill_mfma_kernel(const AttnPrefillParams p) {
  constexpr int BQ = 128, BKV = 64;
  constexpr int LDK = D + 8;        // K tile row stride (elements)
  constexpr int LDV = BKV + 8;      // V^T tile row stride (elements)
  constexpr int KS = D / 16;        // k-steps of the score product
  constexpr int DB = D / 32;        // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) bf16 Ks[BKV * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * LDV];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int S = p.S;
  const int qt = (int)gridDim.x - 1 - (int)blockIdx.x;   // longest tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int rep = p.nq / p.nkv;
  const int j = h / rep;
  const int q0 = qt * BQ;
  const int wq0 = q0 + wid * 32;
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
  const float qscale = p.scale * LOG2E_M;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

  const int kend = min(q0 + BQ, S);
  constexpr int KCH = BKV * D / 8;            // 16-byte chunks per tile
  for (int k0 = 0; k0 < kend; k0 += BKV) {
    __syncthreads();                          // previous tile fully consumed
    // K: coalesced rows;  V: lanes take consecutive keys so the transposed
    // 2-byte LDS writes of one instruction land in consecutive halfwords
#pragma unroll
    for (int i = 0; i < KCH / 256; ++i) {
      const int id = tid + 256 * i;
      {
        const int key = id / (D / 8), c8 = (id % (D / 8)) * 8;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (k0 + key < S) v = *reinterpret_cast<const u32x4*>(kg + (size_t)(k0 + key) * D + c8);
        *reinterpret_cast<u32x4*>(&Ks[key * LDK + c8]) = v;
      }
      {
        const int key = id % BKV, c8 = (id / BKV) * 8;
        bf16x8 v;
        if (k0 + key < S) {
          v = *reinterpret_cast<const bf16x8*>(vg + (size_t)(k0 + key) * D + c8);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) Vt[(c8 + e) * LDV + key] = v[e];
      }
    }
    __syncthreads();
    if (k0 > wq0 + 31) continue;              // every query of this wave precedes the tile

    // ---- S^T for keys k0 + 32*kb + (8*(r/4) + 4*half + r%4), query myq
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + col) * LDK + ks * 16 + half * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // ---- scale, causal mask, online softmax (base 2)
    const bool diag = (k0 + BKV - 1 > wq0);   // tile reaches past some query of this wave
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
        float v = s[kb][r] * qscale;
        if (diag && (key > myq || key >= S)) v = -INFINITY;
        s[kb][r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m_run, mt);        // finite: key 0 <= every query, seen in tile 0
    const float corr = exp2f(m_run - mn);
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(s[kb][r] - mn);
        s[kb][r] = e;
        ls += e;
      }
    ls += __shfl_xor(ls, 32);
    l_run = l_run * corr + ls;
    m_run = mn;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= corr;

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

hipError_t attn_prefill(const AttnPrefillParams& p, hipStream_t s) {
  if (p.B <= 0 || p.S <= 0) return hipSuccess;
  const bool bf = p.q_dt == DT_BF16 && p.kv_dt == DT_BF16 && p.o_dt == DT_BF16;
  if (!bf || (p.d != 128 && p.d != 64)) return attn_prefill_vec(p, s);
  const dim3 grid((p.S + 127) / 128, p.nq, p.B);
  if (p.d == 128)
    attn_prefill_mfma_kernel<128><<<grid, 256, 0, s>>>(p);
  else
    attn_prefill_mfma_kernel<64><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace fsk
