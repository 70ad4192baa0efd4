// Batch-1 decode step as one persistent kernel (0.6B shape: hidden 1024, 16
// query / 8 KV heads of 128, ffn 3072, bf16 weights and KV cache).
//
// What it computes is the step of "Milestones", M4 (one new token against the
// KV cache) through the whole pass of "Coming back to Failed Star", Second
// sitting (embedding, the blocks, final norm, tied head, greedy selection by
// the rule of its section "Next").  A decode step at batch 1 is a chain of
// small dependent products (about six per layer); launched one kernel per
// product, every link pays a launch and a first memory round trip, and the
// weight stream stops at each boundary.  Here one launch runs the whole step:
//
// * 256 workgroups, one per CU, in 8 groups of 32 (workgroup b: group b % 8,
//   rank b / 8; workgroups are dealt to the 8 XCDs round-robin, so a group
//   shares an XCD).  Group j owns KV head j: its Q/K/V rows, the attention of
//   query heads 2j and 2j+1 over the context, and their merge.  The output,
//   gate/up and down projections are split by output rows over all 256.
// * Each workgroup has 8 compute waves and one control wave.  The compute
//   waves hold their weight slice of every projection in registers and
//   request the next layer's slice right after using the current one, so the
//   weight stream runs a whole layer ahead of the dependency chain; they never
//   wait on other workgroups.  The control wave does all cross-workgroup
//   waiting: it polls the exchange records the step needs next, copies them
//   into LDS and releases the compute waves with a workgroup barrier.
//   (Vector loads complete in order per wave, so a wave with weight loads in
//   flight could not poll quickly; the split keeps the two apart.)
// * Exchanges are records of 16 bytes {v0, tag, v1, tag}, written and read with
//   device-coherent (sc1) buffer stores and loads.  The tag names the step,
//   layer and exchange; a reader waits until every record it needs carries
//   the expected tag, so no separate flag or fence is needed, and a record
//   read half-updated shows a stale tag next to the new value.  Buffers are
//   double-buffered by layer parity.
// * Every wait is bounded: past the limit the control wave raises an abort
//   flag (device word and host-mapped word), the workgroup leaves the step,
//   and the host reports the failure at the next call.
//
// Measured (MI355X, 512..768 keys): correct (logits within 2e-6 of the
// multi-kernel path), but slower, ~800 us per step against ~680: each hand-off
// between workgroups costs 2.5-3.5 us in place (a device-coherent poll round
// trip is ~1 us with 256 pollers; the slowest of 32 or 256 producers sets each
// hand-off), about the cost of a kernel boundary in a captured graph (1.6 us
// launch plus a first memory round trip), and the chain has six per layer.  It
// is therefore off by default (FS_DECODE_PERSIST=1 selects it).
//
// Per layer, the hand-offs are: x (all) -> Q/K/V rows (group) -> attention
// partials (group) -> merged attention output (all) -> x after the output
// projection (all) -> SwiGLU output (all) -> x after the down projection.
// Arithmetic follows the multi-kernel path: fp32 activations, fp32
// accumulation, q/k RMSNorm + rotate-half RoPE, the new token's k and v
// rounded to bf16 as the cache stores them, base-2 online softmax.
#include "common.h"
#include "kernels.h"

namespace fsk {

namespace {

constexpr int PH = 1024, PNQ = 16, PNKV = 8, PD = 128, PI = 3072;
constexpr int PG = 8, PR = 32, PNB = PG * PR;       // groups, ranks, workgroups
constexpr int PCW = 8;                              // compute waves
constexpr int PTHREADS = (PCW + 1) * 64;
constexpr int PQROWS = 512 / PR;                    // Q/K/V rows per workgroup (16)
constexpr int POROWS = PH / PNB;                    // output / down rows per workgroup (4)
constexpr int PFEAT = PI / PNB;                     // SwiGLU features per workgroup (12)

// exchange layout, in 16-byte records
constexpr int RX = PH / 2;                          // x or x_mid: 512
constexpr int RQKV = 512 / 2;                       // one group's q|q|k|v: 256
constexpr int RPART = 1 + PD / 2;                   // one (producer, head) partial: 65
constexpr int RATT = PNQ * PD / 2;                  // attention output: 1024
constexpr int RH = PI / 2;                          // SwiGLU output: 1536
constexpr int OFF_X = 0;
constexpr int OFF_QKV = OFF_X + 2 * RX;
constexpr int OFF_PART = OFF_QKV + 2 * PG * RQKV;
constexpr int OFF_ATT = OFF_PART + 2 * PG * PR * 2 * RPART;
constexpr int OFF_XM = OFF_ATT + 2 * RATT;
constexpr int OFF_H = OFF_XM + 2 * RX;
constexpr int OFF_BEST = OFF_H + 2 * RH;
constexpr int OFF_ABORT = OFF_BEST + PNB;            // one record: the abort word
constexpr int EX_RECORDS = OFF_ABORT + 1;

constexpr unsigned SPIN_LIMIT = 1u << 21;           // polls before a wait gives up (~1 s)
constexpr int CACHE_SC1 = 16;                       // buffer cache policy: device scope

enum Hop { HOP_X = 0, HOP_QKV = 1, HOP_PART = 2, HOP_ATT = 3, HOP_XM = 4, HOP_H = 5, HOP_BEST = 6 };

__device__ __forceinline__ unsigned tag_of(unsigned step_tag, int layer, int hop) {
  return step_tag | ((unsigned)layer << 3) | (unsigned)hop;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ex_rsrc(void* ex) {
  return __builtin_amdgcn_make_buffer_rsrc(ex, (short)0, EX_RECORDS * 16, 0x00020000);
}
__device__ __forceinline__ u32x4 rec_load(__amdgpu_buffer_rsrc_t rs, int rec) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, rec * 16, 0, CACHE_SC1);
}
__device__ __forceinline__ void rec_store(__amdgpu_buffer_rsrc_t rs, int rec, float v0, float v1, unsigned tag) {
  const u32x4 r = {__float_as_uint(v0), tag, __float_as_uint(v1), tag};
  __builtin_amdgcn_raw_buffer_store_b128(r, rs, rec * 16, 0, CACHE_SC1);
}

// Workgroup barrier that waits only for this wave's LDS traffic: the weight
// loads in flight stay in flight (a plain __syncthreads would wait for them).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Measurement trace (optional): workgroup 0 records the real-time clock
// (100 MHz) at fixed points, slot = owner * 512 + index.
__device__ __forceinline__ void stamp(long long* trace, int slot) {
  if (trace != nullptr) trace[slot] = (long long)__builtin_amdgcn_s_memrealtime();
}

// dot of 8 bf16 (packed in a u32x4) with 8 floats
__device__ __forceinline__ float dot8(const u32x4 w, const float* a, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(__uint_as_float(w[i] << 16), a[2 * i], acc);
    acc = fmaf(__uint_as_float(w[i] & 0xffff0000u), a[2 * i + 1], acc);
  }
  return acc;
}
__device__ __forceinline__ void lds8(const float* p, float* o) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
  o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
}
__device__ __forceinline__ u32x4 ldw(const bf16* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }

struct Lds {
  float xs[PH];          // residual x entering the layer
  float xm[PH];          // x after the output projection
  float ga[PH], gm[PH];  // input / post-attention norm weights of the layer (final norm for the head)
  float gq[PD], gk[PD];  // q / k norm weights
  float qkv[4 * PD];     // q0', q1' (normalised, rotated, pre-scaled), k' and v as the cache holds them
  float att[PNQ * PD];   // merged attention output
  float hb[PI];          // SwiGLU output
  float wst[PCW][2][2 + PD];   // per compute wave: (m, l, o[128]) of both query heads
  float hloc[PFEAT];     // this workgroup's SwiGLU outputs
  float bestv[PCW];
  int besti[PCW];
  int abort_flag;
  int pad[3];
};

}  // namespace

template <int KPG>
__global__ __launch_bounds__(PTHREADS) void decode_persist_kernel(const DecodePersistParams p) {
  __shared__ Lds S;
  // pad the workgroup's LDS to more than half a CU so one workgroup runs per CU
  __shared__ char lds_pad[96 * 1024 - sizeof(Lds) > 0 ? 96 * 1024 - sizeof(Lds) : 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x, grp = b % PG, rank = b / PG;
  const __amdgpu_buffer_rsrc_t rs = ex_rsrc(p.ex);
  const bf16* __restrict__ E = static_cast<const bf16*>(p.embed);
  const bf16* __restrict__ Wqkv = static_cast<const bf16*>(p.wqkv0);
  const bf16* __restrict__ Wo = static_cast<const bf16*>(p.wo0);
  const bf16* __restrict__ Wgu = static_cast<const bf16*>(p.wgu0);
  const bf16* __restrict__ Wdn = static_cast<const bf16*>(p.wdown0);
  bf16* __restrict__ Kc = static_cast<bf16*>(p.kcache);
  bf16* __restrict__ Vc = static_cast<bf16*>(p.vcache);
  const int n = p.pos + 1;                         // keys after this step
  const int C = p.chunk;                           // keys per workgroup of the group
  const int L = p.n_layers;
  if (tid == 0) S.abort_flag = 0;
  if (b == 0 && tid == 0) lds_pad[0] = 0;
  long long* const tr = (b == 0 && lane == 0) ? p.trace : nullptr;   // control: 0.., compute wave 0: 512..

  if (wave == 0) {
    // ================================================================ control wave
    unsigned spins = 0;
    bool ok = true;
    // waits for records rec0 .. rec0 + N - 1 carrying `tag`; their values go to dst (2 per record)
    auto poll = [&](int rec0, int N, unsigned tag, float* dst) -> bool {
      if (!ok) return false;
      const int per = (N + 63) / 64;
      for (int i0 = 0; i0 < per; i0 += 8) {
        unsigned pending = 0;
        for (int i = 0; i < 8 && i0 + i < per; ++i)
          if (lane + 64 * (i0 + i) < N) pending |= 1u << i;
        while (true) {
          u32x4 r[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int k = min(lane + 64 * (i0 + i), N - 1);
            r[i] = rec_load(rs, rec0 + k);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if ((pending >> i) & 1u) {
              if (r[i][1] == tag && r[i][3] == tag) {
                const int k = lane + 64 * (i0 + i);
                dst[2 * k] = __uint_as_float(r[i][0]);
                dst[2 * k + 1] = __uint_as_float(r[i][2]);
                pending &= ~(1u << i);
              }
            }
          }
          if (__ballot(pending != 0) == 0) break;
          if (++spins > SPIN_LIMIT || ((spins & 63) == 0 && rec_load(rs, OFF_ABORT)[0] != 0)) {
            ok = false;
            if (lane == 0) {
              rec_store(rs, OFF_ABORT, __uint_as_float(1u), 0.f, 1u);
              *p.abort_host = 1;
              S.abort_flag = 1;
            }
            return false;
          }
        }
      }
      return true;
    };
    auto load_norms = [&](int l) {
      const float* ga = p.attn_norm0 + (size_t)l * p.nstride;
      const float* gm = p.mlp_norm0 + (size_t)l * p.nstride;
      for (int k = lane; k < PH / 4; k += 64) {
        reinterpret_cast<f32x4*>(S.ga)[k] = reinterpret_cast<const f32x4*>(ga)[k];
        reinterpret_cast<f32x4*>(S.gm)[k] = reinterpret_cast<const f32x4*>(gm)[k];
      }
      const float* gq = p.q_norm0 + (size_t)l * p.nstride;
      const float* gk = p.k_norm0 + (size_t)l * p.nstride;
      S.gq[lane] = gq[lane]; S.gq[lane + 64] = gq[lane + 64];
      S.gk[lane] = gk[lane]; S.gk[lane + 64] = gk[lane + 64];
    };

    // ---- embedding row of the token (every workgroup reads it itself)
    {
      const int id = p.tokens[0];
      const bool bad = id < 0 || id >= p.V;
      const bf16* row = E + (size_t)(bad ? 0 : id) * PH;
      for (int k = lane; k < PH / 8; k += 64) {
        float v[8];
        load8(row + 8 * k, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) S.xs[8 * k + e] = bad ? __int_as_float(0x7fc00000) : v[e];
      }
      if (bad && b == 0 && lane == 0 && p.tokerr != nullptr) {
        p.tokerr[1] = id;
        p.tokerr[2] = 0;
        __threadfence_system();
        p.tokerr[0] = 1;
      }
      load_norms(0);
    }
    // RoPE angles of this position, shared by every layer
    const float cs = p.cos_t[(size_t)p.pos * (PD / 2) + lane];
    const float sn = p.sin_t[(size_t)p.pos * (PD / 2) + lane];
    const int owner = p.pos / C;                     // the rank whose chunk holds the new key
    stamp(tr, 0);
    wg_barrier();                                    // B0 of layer 0

    for (int l = 0; l < L; ++l) {
      const int par = l & 1;
      // ---- H2: this group's q|q|k|v rows
      const unsigned sp0 = spins;
      ok = poll(OFF_QKV + (par * PG + grp) * RQKV, RQKV, tag_of(p.step_tag, l, HOP_QKV), S.qkv) && ok;
      stamp(tr, 1 + 8 * l);
      if (tr != nullptr) tr[7 + 8 * l] = spins - sp0;          // polls this wait took
      if (ok) {
        // q/k RMSNorm over the head, rotate-half RoPE (lane holds dims lane, lane + 64:
        // a rotation pair), q pre-scaled by scale * log2(e); k and v rounded to bf16
        float kv_k[2], kv_v[2];
#pragma unroll
        for (int h = 0; h < 3; ++h) {
          const float a0 = S.qkv[h * PD + lane], a1 = S.qkv[h * PD + lane + 64];
          const float inv = rsqrtf(wave_sum(fmaf(a0, a0, a1 * a1)) / (float)PD + p.eps);
          const float* g = h < 2 ? S.gq : S.gk;
          const float a = a0 * inv * g[lane], c = a1 * inv * g[lane + 64];
          float y0 = a * cs - c * sn, y1 = c * cs + a * sn;
          if (h < 2) {
            y0 *= p.qscale; y1 *= p.qscale;
          } else {
            y0 = (float)(bf16)y0; y1 = (float)(bf16)y1;
            kv_k[0] = y0; kv_k[1] = y1;
          }
          S.qkv[h * PD + lane] = y0;
          S.qkv[h * PD + lane + 64] = y1;
        }
        const float v0 = (float)(bf16)S.qkv[3 * PD + lane], v1 = (float)(bf16)S.qkv[3 * PD + lane + 64];
        S.qkv[3 * PD + lane] = v0;
        S.qkv[3 * PD + lane + 64] = v1;
        kv_v[0] = v0; kv_v[1] = v1;
        if (rank == owner) {                         // append k, v to the cache at pos
          const size_t o = (size_t)l * p.layer_stride + (size_t)p.slot * p.slot_stride +
                           (size_t)grp * p.head_stride + (size_t)p.pos * PD;
          Kc[o + lane] = (bf16)kv_k[0]; Kc[o + lane + 64] = (bf16)kv_k[1];
          Vc[o + lane] = (bf16)kv_v[0]; Vc[o + lane + 64] = (bf16)kv_v[1];
        }
      }
      if (!ok && lane == 0) S.abort_flag = 1;
      wg_barrier();                                  // B1: q, k, v in LDS
      wg_barrier();                                  // B2: the compute waves' attention states in LDS
      // ---- H3: merge dims [8q, 8q + 8) of head hh of the group over its 32 partials
      {
        const int hh = rank >> 4, q8 = rank & 15;
        const unsigned tg = tag_of(p.step_tag, l, HOP_PART);
        const int base = OFF_PART + (par * PG + grp) * PR * 2 * RPART;
        float mv = -INFINITY, lv = 0.f, ov[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (ok) {
          const int prod = lane & 31;
          const int pb = base + (prod * 2 + hh) * RPART;
          int pending = 1;
          while (true) {
            const u32x4 r0 = rec_load(rs, pb);
            const u32x4 r1 = rec_load(rs, pb + 1 + 4 * q8);
            const u32x4 r2 = rec_load(rs, pb + 2 + 4 * q8);
            const u32x4 r3 = rec_load(rs, pb + 3 + 4 * q8);
            const u32x4 r4 = rec_load(rs, pb + 4 + 4 * q8);
            if (pending && r0[1] == tg && r0[3] == tg && r1[1] == tg && r1[3] == tg && r2[1] == tg &&
                r2[3] == tg && r3[1] == tg && r3[3] == tg && r4[1] == tg && r4[3] == tg) {
              mv = __uint_as_float(r0[0]); lv = __uint_as_float(r0[2]);
              ov[0] = __uint_as_float(r1[0]); ov[1] = __uint_as_float(r1[2]);
              ov[2] = __uint_as_float(r2[0]); ov[3] = __uint_as_float(r2[2]);
              ov[4] = __uint_as_float(r3[0]); ov[5] = __uint_as_float(r3[2]);
              ov[6] = __uint_as_float(r4[0]); ov[7] = __uint_as_float(r4[2]);
              pending = 0;
            }
            if (__ballot(pending != 0) == 0) break;
            if (++spins > SPIN_LIMIT || ((spins & 63) == 0 && rec_load(rs, OFF_ABORT)[0] != 0)) {
              ok = false;
              if (lane == 0) {
                rec_store(rs, OFF_ABORT, __uint_as_float(1u), 0.f, 1u);
                *p.abort_host = 1;
                S.abort_flag = 1;
              }
              break;
            }
          }
        }
        if (lane >= 32) { mv = -INFINITY; lv = 0.f; }   // the upper half holds copies
        const float M = wave_max(mv);
        const float a = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
        const float Ls = wave_sum(a * lv);
        float outv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) outv[k] = wave_sum(a * ov[k]) / Ls;
        if (ok && lane < 4) {
          // query head of this merge: 2 * grp + hh; its dims [8 q8, 8 q8 + 8)
          const int dim0 = (2 * grp + hh) * PD + 8 * q8 + 2 * lane;
          const float w0 = lane == 0 ? outv[0] : lane == 1 ? outv[2] : lane == 2 ? outv[4] : outv[6];
          const float w1 = lane == 0 ? outv[1] : lane == 1 ? outv[3] : lane == 2 ? outv[5] : outv[7];
          rec_store(rs, OFF_ATT + par * RATT + dim0 / 2, w0, w1, tag_of(p.step_tag, l, HOP_ATT));
        }
      }
      stamp(tr, 2 + 8 * l);
      // ---- H4: the whole attention output
      ok = poll(OFF_ATT + par * RATT, RATT, tag_of(p.step_tag, l, HOP_ATT), S.att) && ok;
      stamp(tr, 3 + 8 * l);
      if (!ok && lane == 0) S.abort_flag = 1;
      wg_barrier();                                  // B3: attention output in LDS
      // ---- H5: x after the output projection
      ok = poll(OFF_XM + par * RX, RX, tag_of(p.step_tag, l, HOP_XM), S.xm) && ok;
      stamp(tr, 4 + 8 * l);
      if (!ok && lane == 0) S.abort_flag = 1;
      wg_barrier();                                  // B5: x_mid in LDS
      wg_barrier();                                  // B6: this workgroup's SwiGLU outputs in LDS
      if (ok && lane < PFEAT / 2) {
        rec_store(rs, OFF_H + par * RH + b * (PFEAT / 2) + lane, S.hloc[2 * lane], S.hloc[2 * lane + 1],
                  tag_of(p.step_tag, l, HOP_H));
      }
      // ---- H6: the whole SwiGLU output
      ok = poll(OFF_H + par * RH, RH, tag_of(p.step_tag, l, HOP_H), S.hb) && ok;
      stamp(tr, 5 + 8 * l);
      if (!ok && lane == 0) S.abort_flag = 1;
      wg_barrier();                                  // B7: SwiGLU output in LDS
      // ---- H1 of the next layer: x after the down projection
      ok = poll(OFF_X + ((l + 1) & 1) * RX, RX, tag_of(p.step_tag, l + 1, HOP_X), S.xs) && ok;
      stamp(tr, 6 + 8 * l);
      if (l + 1 < L) load_norms(l + 1);
      else {
        for (int k = lane; k < PH / 4; k += 64)
          reinterpret_cast<f32x4*>(S.ga)[k] = reinterpret_cast<const f32x4*>(p.final_norm)[k];
      }
      if (!ok && lane == 0) S.abort_flag = 1;
      wg_barrier();                                  // B0 of the next layer (or of the head)
    }
    wg_barrier();                                    // BH: the compute waves' head bests in LDS
    if (ok) {
      float bv = S.bestv[0];
      int bi = S.besti[0];
      for (int w = 1; w < PCW; ++w)
        if (better(S.bestv[w], S.besti[w], bv, bi)) { bv = S.bestv[w]; bi = S.besti[w]; }
      const unsigned tg = tag_of(p.step_tag, L, HOP_BEST);
      if (lane == 0) rec_store(rs, OFF_BEST + b, bv, __int_as_float(bi), tg);
      if (b == 0 && p.next != nullptr) {
        poll(OFF_BEST, PNB, tg, S.hb);
        float v = 0.f;
        int i = -1;
#pragma unroll
        for (int k = 0; k < PNB / 64; ++k) {
          const float cv = S.hb[2 * (lane + 64 * k)];
          const int ci = __float_as_int(S.hb[2 * (lane + 64 * k) + 1]);
          if (better(cv, ci, v, i)) { v = cv; i = ci; }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ov = __shfl_xor(v, o);
          const int oi = __shfl_xor(i, o);
          if (better(ov, oi, v, i)) { v = ov; i = oi; }
        }
        if (lane == 0 && ok) p.next[0] = i;
        stamp(tr, 511);
      }
    }
    return;
  }

  // ================================================================== compute waves
  const int cw = wave - 1;
  const int li = lane & 15, grp4 = lane >> 4;     // attention: 16-lane group, its 8 dims
  // this workgroup's Q/K/V rows: 8 ranks per section (q head 2j, q head 2j+1, k head j, v head j)
  const int sec = rank >> 3, srow = (rank & 7) * PQROWS;
  const int qrow0 = (sec < 2 ? grp * 2 * PD + sec * PD : sec == 2 ? PNQ * PD + grp * PD : (PNQ + PNKV) * PD + grp * PD) + srow;
  // roles in the output / SwiGLU / down projections
  const int orow = POROWS * b + 2 * cw;           // cw 0, 1: output rows orow, orow + 1
  const int drow = POROWS * b + 2 * (cw - 2);     // cw 2, 3: down rows
  const int f0 = PFEAT * b + 3 * (cw - 4);        // cw 4..7: features f0 .. f0 + 2
  // key slots: slot s = kk * 32 + cw * 4 + grp4 of the workgroup's chunk [rank * C, rank * C + C)
  const int kbase = rank * C;

  u32x4 wq[2][2];             // Q/K/V rows 2cw, 2cw + 1 of the slice, chunks lane, lane + 64
  u32x4 wr[12];               // output rows (8 used) / gate,up rows (12) / down rows (12)
  u32x4 kr[KPG], vr[KPG];     // K/V rows of this lane group's key slots, dims [8 li, 8 li + 8)

  auto load_layer_qkv = [&](int l) {
    const bf16* w = Wqkv + (size_t)l * p.wstride;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) wq[i][c] = ldw(w + (size_t)(qrow0 + 2 * cw + i) * PH + 8 * (lane + 64 * c));
  };
  auto load_layer_kv = [&](int l) {
    const size_t o = (size_t)l * p.layer_stride + (size_t)p.slot * p.slot_stride + (size_t)grp * p.head_stride;
    const int last = max(p.pos - 1, 0);           // the cache holds positions 0 .. pos - 1
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      const int key = min(kbase + kk * 32 + cw * 4 + grp4, last);
      kr[kk] = ldw(Kc + o + (size_t)key * PD + 8 * li);
      vr[kk] = ldw(Vc + o + (size_t)key * PD + 8 * li);
    }
  };
  auto load_layer_rest = [&](int l) {
    if (cw < 2) {
      const bf16* w = Wo + (size_t)l * p.wstride;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) wr[i * 4 + c] = ldw(w + (size_t)(orow + i) * (PNQ * PD) + 8 * (lane + 64 * c));
#pragma unroll
      for (int k = 8; k < 12; ++k) wr[k] = wr[k - 8];
    } else if (cw < 4) {
      const bf16* w = Wdn + (size_t)l * p.wstride;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < 6; ++c) wr[i * 6 + c] = ldw(w + (size_t)(drow + i) * PI + 8 * (lane + 64 * c));
    } else {
      const bf16* w = Wgu + (size_t)l * p.wstride;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int f = f0 + k;
        const int gr = (f >> 5) * 64 + (f & 31);      // packed: 32 gate rows then the matching 32 up rows
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < 2; ++c) wr[(k * 2 + u) * 2 + c] = ldw(w + (size_t)(gr + 32 * u) * PH + 8 * (lane + 64 * c));
      }
    }
  };
  load_layer_qkv(0);
  load_layer_kv(0);
  load_layer_rest(0);
  wg_barrier();                                     // B0 of layer 0: x in LDS

  long long* const tc = (cw == 0) ? tr : nullptr;
  for (int l = 0; l < L; ++l) {
    if (S.abort_flag) return;
    const int par = l & 1;
    const int ln = min(l + 1, L - 1);               // the layer whose weights go in flight next
    stamp(tc, 512 + 8 * l);
    // ---------------------------------------------------------- Q/K/V rows
    {
      float xa[2][8];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        lds8(S.xs + 8 * (lane + 64 * c), xa[c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(xa[c][e], xa[c][e], ss);
      }
      const float inv = rsqrtf(wave_sum(ss) / (float)PH + p.eps);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float g[8];
        lds8(S.ga + 8 * (lane + 64 * c), g);
#pragma unroll
        for (int e = 0; e < 8; ++e) xa[c][e] = xa[c][e] * inv * g[e];
      }
      float y[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) y[i] = wave_sum(dot8(wq[i][1], xa[1], dot8(wq[i][0], xa[0], 0.f)));
      load_layer_qkv(ln);
      if (lane == 0)
        rec_store(rs, OFF_QKV + (par * PG + grp) * RQKV + (sec * PD + srow) / 2 + cw, y[0], y[1],
                  tag_of(p.step_tag, l, HOP_QKV));
    }
    stamp(tc, 513 + 8 * l);
    wg_barrier();                                   // B1
    if (S.abort_flag) return;
    stamp(tc, 514 + 8 * l);
    // ---------------------------------------------------------- attention over this workgroup's keys
    {
      float q0[8], q1[8], kn[8], vn[8];
      lds8(S.qkv + 8 * li, q0);
      lds8(S.qkv + PD + 8 * li, q1);
      lds8(S.qkv + 2 * PD + 8 * li, kn);
      lds8(S.qkv + 3 * PD + 8 * li, vn);
      float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.f, l1 = 0.f, o0[8], o1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { o0[e] = 0.f; o1[e] = 0.f; }
#pragma unroll
      for (int kk = 0; kk < KPG; ++kk) {
        const int slot_i = kk * 32 + cw * 4 + grp4;
        const int key = kbase + slot_i;
        const bool valid = slot_i < C && key < n;
        const bool isnew = key == p.pos;
        float kf[8], vf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kf[2 * i] = __uint_as_float(kr[kk][i] << 16);
          kf[2 * i + 1] = __uint_as_float(kr[kk][i] & 0xffff0000u);
          vf[2 * i] = __uint_as_float(vr[kk][i] << 16);
          vf[2 * i + 1] = __uint_as_float(vr[kk][i] & 0xffff0000u);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kf[e] = isnew ? kn[e] : kf[e];
          vf[e] = isnew ? vn[e] : vf[e];
        }
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { s0 = fmaf(q0[e], kf[e], s0); s1 = fmaf(q1[e], kf[e], s1); }
        s0 = row16_sum(s0);
        s1 = row16_sum(s1);
        if (valid) {
          const float n0 = fmaxf(m0, s0), n1 = fmaxf(m1, s1);
          const float c0 = __builtin_amdgcn_exp2f(m0 - n0), c1 = __builtin_amdgcn_exp2f(m1 - n1);
          const float p0 = __builtin_amdgcn_exp2f(s0 - n0), p1 = __builtin_amdgcn_exp2f(s1 - n1);
          l0 = l0 * c0 + p0;
          l1 = l1 * c1 + p1;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            o0[e] = fmaf(p0, vf[e], o0[e] * c0);
            o1[e] = fmaf(p1, vf[e], o1[e] * c1);
          }
          m0 = n0;
          m1 = n1;
        }
      }
      load_layer_kv(ln);
      // merge the wave's four 16-lane groups
      auto merge = [&](float& m, float& lsum, float* o, auto other) {
        const float mo = other(m), lo = other(lsum);
        const float mn = fmaxf(m, mo);
        const float a = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float c = (mo == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
        lsum = lsum * a + lo * c;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = o[e] * a + other(o[e]) * c;
        m = mn;
      };
      auto x16 = [](float v) { return xor16_f(v); };
      auto x32 = [](float v) { return xor32_f(v); };
      merge(m0, l0, o0, x16); merge(m1, l1, o1, x16);
      merge(m0, l0, o0, x32); merge(m1, l1, o1, x32);
      if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          S.wst[cw][0][2 + 8 * li + e] = o0[e];
          S.wst[cw][1][2 + 8 * li + e] = o1[e];
        }
        if (lane == 0) {
          S.wst[cw][0][0] = m0; S.wst[cw][0][1] = l0;
          S.wst[cw][1][0] = m1; S.wst[cw][1][1] = l1;
        }
      }
    }
    stamp(tc, 515 + 8 * l);
    wg_barrier();                                   // B2
    if (cw < 2) {
      // the workgroup's partial of head cw: (m, l, o[128]) over its keys
      const int h = cw;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < PCW; ++w) M = fmaxf(M, S.wst[w][h][0]);
      float Ls = 0.f, oa = 0.f, ob = 0.f;
#pragma unroll
      for (int w = 0; w < PCW; ++w) {
        const float mw = S.wst[w][h][0];
        const float a = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        Ls = fmaf(a, S.wst[w][h][1], Ls);
        oa = fmaf(a, S.wst[w][h][2 + 2 * lane], oa);
        ob = fmaf(a, S.wst[w][h][3 + 2 * lane], ob);
      }
      const int pb = OFF_PART + ((par * PG + grp) * PR * 2 + rank * 2 + h) * RPART;
      const unsigned tg = tag_of(p.step_tag, l, HOP_PART);
      rec_store(rs, pb + 1 + lane, oa, ob, tg);
      if (lane == 0) rec_store(rs, pb, M, Ls, tg);
    }
    wg_barrier();                                   // B3
    if (S.abort_flag) return;
    // ---------------------------------------------------------- output projection rows (+ residual)
    if (cw < 2) {
      float y[2] = {0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float a[8];
        lds8(S.att + 8 * (lane + 64 * c), a);
#pragma unroll
        for (int i = 0; i < 2; ++i) y[i] = dot8(wr[i * 4 + c], a, y[i]);
      }
      y[0] = wave_sum(y[0]);
      y[1] = wave_sum(y[1]);
      const float x0 = S.xs[orow] + y[0], x1 = S.xs[orow + 1] + y[1];
      load_layer_rest(ln);
      if (lane == 0) rec_store(rs, OFF_XM + par * RX + orow / 2, x0, x1, tag_of(p.step_tag, l, HOP_XM));
      stamp(tc, 516 + 8 * l);
    }
    wg_barrier();                                   // B5
    if (S.abort_flag) return;
    // ---------------------------------------------------------- gate/up + SwiGLU
    if (cw >= 4) {
      float xa[2][8];
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        lds8(S.xm + 8 * (lane + 64 * c), xa[c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(xa[c][e], xa[c][e], ss);
      }
      const float inv = rsqrtf(wave_sum(ss) / (float)PH + p.eps);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float g[8];
        lds8(S.gm + 8 * (lane + 64 * c), g);
#pragma unroll
        for (int e = 0; e < 8; ++e) xa[c][e] = xa[c][e] * inv * g[e];
      }
      float hv[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float yg = wave_sum(dot8(wr[(k * 2) * 2 + 1], xa[1], dot8(wr[(k * 2) * 2], xa[0], 0.f)));
        const float yu = wave_sum(dot8(wr[(k * 2 + 1) * 2 + 1], xa[1], dot8(wr[(k * 2 + 1) * 2], xa[0], 0.f)));
        hv[k] = silu(yg) * yu;
      }
      load_layer_rest(ln);
      if (lane == 0) {
#pragma unroll
        for (int k = 0; k < 3; ++k) S.hloc[3 * (cw - 4) + k] = hv[k];
      }
    }
    wg_barrier();                                   // B6
    wg_barrier();                                   // B7
    if (S.abort_flag) return;
    // ---------------------------------------------------------- down projection rows (+ residual)
    if (cw >= 2 && cw < 4) {
      float y[2] = {0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 6; ++c) {
        float a[8];
        lds8(S.hb + 8 * (lane + 64 * c), a);
#pragma unroll
        for (int i = 0; i < 2; ++i) y[i] = dot8(wr[i * 6 + c], a, y[i]);
      }
      y[0] = wave_sum(y[0]);
      y[1] = wave_sum(y[1]);
      const float x0 = S.xm[drow] + y[0], x1 = S.xm[drow + 1] + y[1];
      load_layer_rest(ln);
      if (lane == 0)
        rec_store(rs, OFF_X + ((l + 1) & 1) * RX + drow / 2, x0, x1, tag_of(p.step_tag, l + 1, HOP_X));
    }
    wg_barrier();                                   // B0 of the next layer
  }
  if (S.abort_flag) return;
  // ------------------------------------------------------------ final RMSNorm + tied head (+ argmax)
  {
    float xa[2][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      lds8(S.xs + 8 * (lane + 64 * c), xa[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(xa[c][e], xa[c][e], ss);
    }
    const float inv = rsqrtf(wave_sum(ss) / (float)PH + p.eps);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float g[8];
      lds8(S.ga + 8 * (lane + 64 * c), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) xa[c][e] = xa[c][e] * inv * g[e];
    }
    const int rpb = (p.V + PNB - 1) / PNB;
    const int r0 = b * rpb, r1 = min(p.V, r0 + rpb);
    float bv = 0.f;
    int bi = -1;
    constexpr int G = 4;                              // rows per group; two groups in flight
    u32x4 ra[G][2], rb[G][2];
    auto load_rows = [&](int g, u32x4 (&r)[G][2]) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int row = min(r0 + (g * G + i) * PCW + cw, r1 - 1);
#pragma unroll
        for (int c = 0; c < 2; ++c) r[i][c] = ldw(E + (size_t)row * PH + 8 * (lane + 64 * c));
      }
    };
    auto use_rows = [&](int g, const u32x4 (&r)[G][2]) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int row = r0 + (g * G + i) * PCW + cw;
        const float v = wave_sum(dot8(r[i][1], xa[1], dot8(r[i][0], xa[0], 0.f)));
        if (row < r1) {
          if (p.logits != nullptr && lane == 0) p.logits[row] = v;
          if (__builtin_isfinite(v) && better(v, row, bv, bi)) { bv = v; bi = row; }
        }
      }
    };
    const int ng = (rpb + G * PCW - 1) / (G * PCW);   // groups per wave (even count below)
    const int ng2 = (ng + 1) & ~1;
    load_rows(0, ra);
#pragma unroll 1
    for (int g = 0; g < ng2; g += 2) {
      load_rows(g + 1, rb);
      use_rows(g, ra);
      load_rows(min(g + 2, ng2 - 1), ra);
      use_rows(g + 1, rb);
    }
    if (lane == 0) { S.bestv[cw] = bv; S.besti[cw] = bi; }
    stamp(tc, 1023);
  }
  wg_barrier();                                     // BH
}

bool decode_persist_ok(int n_layers, int hidden, int n_heads, int n_kv_heads, int head_dim, int ffn, int dt,
                       int wdt, int gated, int rot) {
  return n_layers >= 1 && n_layers < 31 && hidden == PH && n_heads == PNQ && n_kv_heads == PNKV && head_dim == PD && ffn == PI &&
         dt == DT_BF16 && wdt == DT_BF16 && !gated && rot == PD;
}

int decode_persist_max_ctx() { return 2 * 32 * PR; }

size_t decode_persist_exchange_bytes() { return (size_t)EX_RECORDS * 16; }

hipError_t decode_persist(const DecodePersistParams& p, hipStream_t s) {
  if (p.pos < 0 || p.pos + 1 > decode_persist_max_ctx() || p.chunk * PR < p.pos + 1 || p.chunk <= 0)
    return hipErrorInvalidValue;
  const int kpg = (p.chunk + 31) / 32;
  if (kpg == 1)
    decode_persist_kernel<1><<<PNB, PTHREADS, 0, s>>>(p);
  else if (kpg == 2)
    decode_persist_kernel<2><<<PNB, PTHREADS, 0, s>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fsk
