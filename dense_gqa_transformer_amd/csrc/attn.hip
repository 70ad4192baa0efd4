// Grouped-query causal attention over the KV cache (wave64 vector path).
//
// Query head h reads KV head h / (nq/nkv); the query at position p attends to
// keys 0..p inclusive with scores scaled by 1/sqrt(d) and a max-subtracted
// softmax ("Failed Star (fs)", How it's built: GQA; "Coming back to Failed
// Star", Second sitting: 16 query heads and 8 KV heads of width 128).
//
// Work layout: a wave is four groups of 16 lanes; each group walks its own
// key positions, lane i of a group holding elements [i*d/16, (i+1)*d/16) of
// q, k, v.  Each group keeps an online-softmax state (running max m, sum l,
// unnormalised output o) in base 2 (q is pre-scaled by log2(e)/sqrt(d)).
// Group states merge exactly: m = max, l and o rescaled by 2^(m_g - m).
//
// Decode kernel: one workgroup per (sequence, KV head, context chunk).  It
// also normalises and rotates the new token's q and k (rotate-half on the
// first `rot` dims; q rows interleaved with gate rows when the variant is
// gated) and appends k, v to the cache (fused), and writes the chunk's
// partial softmax state; the partials are combined by the consumer (split-K
// flash decoding).  One-pass form, for short contexts at small batch: one
// workgroup of 16 waves per (sequence, KV head) walks the whole context, the
// 16 wave states merge in LDS and the normalised output is written directly,
// which saves the merge launch (a few microseconds) at the price of streaming
// each KV head's context through one CU.
#include "common.h"
#include "kernels.h"

namespace fsk {

static constexpr float LOG2E = 1.4426950408889634f;

template <typename KV, int N> __device__ __forceinline__ void loadn(const KV* p, float* o);
template <> __device__ __forceinline__ void loadn<bf16, 8>(const bf16* p, float* o) { load8(p, o); }
template <> __device__ __forceinline__ void loadn<bf16, 4>(const bf16* p, float* o) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
  o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
}
template <> __device__ __forceinline__ void loadn<float, 8>(const float* p, float* o) { load8(p, o); }
template <> __device__ __forceinline__ void loadn<float, 4>(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
}

template <> __device__ __forceinline__ void loadn<bf16, 16>(const bf16* p, float* o) { load8(p, o); load8(p + 8, o + 8); }
template <> __device__ __forceinline__ void loadn<float, 16>(const float* p, float* o) { load8(p, o); load8(p + 8, o + 8); }

// Raw (unconverted) loads of d/16 elements, so a batch of them can be in
// flight before any is used.
template <typename KV, int N> struct RawKV;
template <> struct RawKV<bf16, 8> {
  u32x4 v;
  // K/V rows are read once per step: streaming (nontemporal) loads
  __device__ __forceinline__ void load(const bf16* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ void get(float* o) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = __uint_as_float(v[i] << 16); o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u); }
  }
};
template <> struct RawKV<bf16, 4> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void get(float* o) const {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};
template <> struct RawKV<float, 8> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p); b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void get(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};
template <> struct RawKV<float, 4> {
  float4 a;
  __device__ __forceinline__ void load(const float* p) { a = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void get(float* o) const { o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; }
};

template <typename KV> struct RawKV<KV, 16> {
  RawKV<KV, 8> a, b;
  __device__ __forceinline__ void load(const KV* p) { a.load(p); b.load(p + 8); }
  __device__ __forceinline__ void get(float* o) const { a.get(o); b.get(o + 8); }
};

// x[e] of the np (1 or 2) split-K partials of the projection, pst floats
// apart, as a pair to be summed once the loads are in (psum).  Both loads are
// issued either way (with one partial the second re-reads x[e]), so the
// number of loads does not depend on np.
struct Part2 {
  float a, b;
};
__device__ __forceinline__ Part2 ld_part(const float* x, size_t pst, int np, int e) {
  return Part2{x[e], x[(np > 1 ? pst : 0) + e]};
}
__device__ __forceinline__ float psum(const Part2& p, int np) { return np > 1 ? p.a + p.b : p.a; }

// RMSNorm over d (weight g) of one head's projection row x (summed over its
// np split-K partials, pst floats apart), then rotate-half RoPE on the first
// `rot` dims (element e < rot/2 pairs with e + rot/2; cos/sin rows of length
// rot/2), times `mul`.  One wave: lane holds elements lane + 64i (returned in
// y[i]).  Split in two so that a kernel can request every load of the step
// (nr_fetch) before other loads, and compute (nr_finish) once they are in.
// A full rotation of two elements per lane has a path of its own (the partner
// is the lane's other element, so half the loads); wider rows take the general
// path for every rotation width: with a second path there the compiler merges
// the two paths' stores into one store at a path-dependent index, which puts
// the struct in scratch memory.
template <int D>
struct NormRopeIn {
  static constexpr int NE = D / 64;
  Part2 v[NE], vp[NE];
  float gv[NE], gp[NE], c[NE], s[NE];
};

template <int D>
__device__ __forceinline__ void nr_fetch(const float* x, size_t pst, int np, const float* g, const float* cs,
                                         const float* sn, int rot, int lane, NormRopeIn<D>& in) {
  constexpr int NE = D / 64;
  const int rh = rot >> 1;
  if constexpr (NE == 2) {
    if (rot == D) {
      // full rotation: element i's partner is element i +- NE/2 of the same lane
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        in.v[i] = ld_part(x, pst, np, lane + 64 * i);
        in.gv[i] = g[lane + 64 * i];
      }
#pragma unroll
      for (int i = 0; i < NE / 2; ++i) {
        in.c[i] = cs[lane + 64 * i];
        in.s[i] = sn[lane + 64 * i];
      }
      return;
    }
  }
  // every load is unconditional (a dim outside the rotation reads angle 0 and
  // ignores it)
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    const bool r = e < rot, lo = e < rh;
    const int pe = r ? (lo ? e + rh : e - rh) : e, fi = r ? (lo ? e : e - rh) : 0;
    in.v[i] = ld_part(x, pst, np, e);
    in.vp[i] = ld_part(x, pst, np, pe);
    in.gv[i] = g[e];
    in.gp[i] = g[pe];
    const float cv = cs[fi], sv = sn[fi];
    in.c[i] = r ? cv : 1.f;
    in.s[i] = r ? (lo ? -sv : sv) : 0.f;
  }
}

template <int D>
__device__ __forceinline__ void nr_finish(const NormRopeIn<D>& in, int np, int rot, float eps, float mul,
                                          float (&y)[D / 64]) {
  constexpr int NE = D / 64;
  float v[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) v[i] = psum(in.v[i], np);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) ss = fmaf(v[i], v[i], ss);
  const float inv = rsqrtf(wave_sum(ss) / (float)D + eps);
  if constexpr (NE == 2) {
    if (rot == D) {
      constexpr int H = NE / 2;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float a = v[i] * inv * in.gv[i], b = v[i + H] * inv * in.gv[i + H];
        y[i] = (a * in.c[i] - b * in.s[i]) * mul;
        y[i + H] = (b * in.c[i] + a * in.s[i]) * mul;
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const float a = v[i] * inv * in.gv[i], b = psum(in.vp[i], np) * inv * in.gp[i];
    y[i] = (a * in.c[i] + b * in.s[i]) * mul;
  }
}

template <int REP, int DP>
struct SoftState {
  float m[REP], l[REP], o[REP][DP];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int r = 0; r < REP; ++r) {
      m[r] = -INFINITY;
      l[r] = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) o[r][e] = 0.f;
    }
  }
  // fold one key position: s[r] = base-2 score, v = this lane's value slice.
  // The reference m only moves when a score exceeds it by more than 2^8 (and
  // on the first position, where m is -inf), so the accumulators are rarely
  // rescaled; l and o use the same m, so the final o / l is unchanged.
  __device__ __forceinline__ void add(const float* s, const float* v) {
#pragma unroll
    for (int r = 0; r < REP; ++r) {
      if (s[r] > m[r] + 8.f) {
        const float corr = __builtin_amdgcn_exp2f(m[r] - s[r]);   // 0 while m is -inf
        l[r] *= corr;
#pragma unroll
        for (int e = 0; e < DP; ++e) o[r][e] *= corr;
        m[r] = s[r];
      }
      const float pp = __builtin_amdgcn_exp2f(s[r] - m[r]);
      l[r] += pp;
#pragma unroll
      for (int e = 0; e < DP; ++e) o[r][e] = fmaf(pp, v[e], o[r][e]);
    }
  }
  // merge with the state held OFF lanes away (xor; 16 or 32)
  template <int OFF>
  __device__ __forceinline__ void merge_xor() {
    static_assert(OFF == 16 || OFF == 32, "row-pair or half-wave exchange");
    auto other = [](float v) { return OFF == 16 ? xor16_f(v) : xor32_f(v); };
#pragma unroll
    for (int r = 0; r < REP; ++r) {
      const float mo = other(m[r]);
      const float lo = other(l[r]);
      const float mn = fmaxf(m[r], mo);
      const float a = (m[r] == -INFINITY) ? 0.f : exp2f(m[r] - mn);
      const float b = (mo == -INFINITY) ? 0.f : exp2f(mo - mn);
      l[r] = l[r] * a + lo * b;
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        const float oo = other(o[r][e]);
        o[r][e] = o[r][e] * a + oo * b;
      }
      m[r] = mn;
    }
  }
};

// Walks positions u = first + 4*i (< end) for this lane's group; uniform trip
// count across the wave so the 16-lane shuffles stay converged.
template <typename KV, int D, int REP>
__device__ __forceinline__ void attend(SoftState<REP, D / 16>& st, const float (&q)[REP][D / 16],
                                       const KV* __restrict__ kb, const KV* __restrict__ vb,
                                       int wave_first, int end, int stride, int grp, int li,
                                       int u_new, const float* knew, const float* vnew) {
  constexpr int DP = D / 16;
  for (int base = wave_first; base < end; base += stride) {
    const int u = base + grp;
    const bool valid = u < end;
    const int uu = valid ? u : wave_first;
    float k[DP], v[DP];
    if (uu == u_new) {
#pragma unroll
      for (int e = 0; e < DP; ++e) { k[e] = knew[li * DP + e]; v[e] = vnew[li * DP + e]; }
    } else {
      loadn<KV, DP>(kb + (size_t)uu * D + li * DP, k);
      loadn<KV, DP>(vb + (size_t)uu * D + li * DP, v);
    }
    float s[REP];
#pragma unroll
    for (int r = 0; r < REP; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) acc = fmaf(q[r][e], k[e], acc);
      s[r] = group_sum<16>(acc);
    }
    if (valid) st.add(s, v);
  }
}

// ------------------------------------------------------------------ decode
// ONE: the one-pass form (16 waves, the whole context, output written to
// p.out); otherwise 4 waves per chunk writing partials.
template <typename KV, int D, int REP, bool ONE>
__global__ __launch_bounds__(ONE ? 1024 : 256) void attn_decode_kernel(const AttnDecodeParams p) {
  constexpr int DP = D / 16;
  constexpr int NW = ONE ? 16 : 4;                      // waves
  constexpr int STEP = 4 * NW;                          // positions per step of the workgroup
  __shared__ float qs[REP][D];
  __shared__ float knew[D], vnew[D];
  __shared__ float sm[NW][REP], sl[NW][REP];
  __shared__ float so[NW][REP][D];

  constexpr int NPRE = 2;                               // key rows per lane in flight
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches below
  const int grp = lane >> 4, li = lane & 15;
  const int pos = p.positions[b];
  const int slot = p.slots[b];
  const int n = pos + 1;
  const int c0 = ONE ? 0 : c * p.chunk;
  if (c0 >= n) return;                                  // chunk past this sequence
  const int c1 = ONE ? n : min(c0 + p.chunk, n);
  const int qmul = p.gated ? 2 : 1;                      // q rows interleaved with gate rows
  const int W = (p.nq * qmul + 2 * p.nkv) * D;
  const float* row = p.qkv + (size_t)b * W;
  const size_t pst = (size_t)p.B * W;                   // between split-K partials of the projection
  const size_t kvoff = (size_t)slot * p.slot_stride + (size_t)j * p.head_stride;
  KV* kb = reinterpret_cast<KV*>(p.kcache) + kvoff;
  KV* vb = reinterpret_cast<KV*>(p.vcache) + kvoff;
  const float qscale = p.scale * LOG2E;
  const bool has_new = (pos >= c0 && pos < c1);

  // ---- every load of the prologue in one round trip, in this order: the q
  //      heads of this wave and (the chunk holding pos, last wave) the new
  //      token's k and v, then this lane's first key/value rows.  The loads
  //      complete in order, so the q/k normalisation waits only for the first
  //      group while the key/value rows are still in flight.  (Row `pos` is
  //      not in the cache yet: it is taken from LDS below.)
  const float* cs_row = p.cos_t + (size_t)pos * (p.rot >> 1);
  const float* sn_row = p.sin_t + (size_t)pos * (p.rot >> 1);
  constexpr int QPW = (REP + NW - 1) / NW;             // q heads per wave, at most
  NormRopeIn<D> qin[QPW];
#pragma unroll
  for (int t = 0; t < QPW; ++t) {
    const int r = wid + NW * t;
    if (r < REP)
      nr_fetch<D>(row + (size_t)(j * REP + r) * D * qmul, pst, p.qkv_np, p.gq, cs_row, sn_row, p.rot, lane, qin[t]);
  }
  const bool do_new = has_new && wid == NW - 1;
  const float* kr = row + (size_t)p.nq * D * qmul + j * D;
  const float* vr = kr + (size_t)p.nkv * D;
  NormRopeIn<D> kin;
  Part2 vv[D / 64];
  if (do_new) {
    nr_fetch<D>(kr, pst, p.qkv_np, p.gk, cs_row, sn_row, p.rot, lane, kin);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) vv[i] = ld_part(vr, pst, p.qkv_np, lane + 64 * i);
  }
  const int ufirst = c0 + wid * 4 + grp;
  RawKV<KV, DP> pk[NPRE], pv[NPRE];
#pragma unroll
  for (int i = 0; i < NPRE; ++i) {
    const int u = min(ufirst + STEP * i, c1 - 1);
    pk[i].load(kb + (size_t)u * D + li * DP);
    pv[i].load(vb + (size_t)u * D + li * DP);
  }

  // ---- q heads: RMSNorm over d, RoPE at pos, pre-scale
#pragma unroll
  for (int t = 0; t < QPW; ++t) {
    const int r = wid + NW * t;
    if (r < REP) {
      float y[D / 64];
      nr_finish<D>(qin[t], p.qkv_np, p.rot, p.eps, qscale, y);
#pragma unroll
      for (int i = 0; i < D / 64; ++i) qs[r][lane + 64 * i] = y[i];
    }
  }
  // ---- the new token's k, v if it falls in this chunk: normalise, rotate, append
  if (do_new) {
    float y[D / 64];
    nr_finish<D>(kin, p.qkv_np, p.rot, p.eps, 1.f, y);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int e = lane + 64 * i;
      const KV kk = from_f32<KV>(y[i]), vk = from_f32<KV>(psum(vv[i], p.qkv_np));
      kb[(size_t)pos * D + e] = kk;
      vb[(size_t)pos * D + e] = vk;
      knew[e] = to_f32(kk);
      vnew[e] = to_f32(vk);
    }
  }
  __syncthreads();

  float q[REP][DP];
#pragma unroll
  for (int r = 0; r < REP; ++r)
#pragma unroll
    for (int e = 0; e < DP; ++e) q[r][e] = qs[r][li * DP + e];

  SoftState<REP, DP> st;
  st.init();
  const int u_new = has_new ? pos : -1;
  auto fold = [&](int u, const float* k, const float* v) {
    float sc[REP];
#pragma unroll
    for (int r = 0; r < REP; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) acc = fmaf(q[r][e], k[e], acc);
      sc[r] = group_sum<16>(acc);
    }
    if (u < c1) st.add(sc, v);
  };
  // positions ufirst + STEP*i, i = 0, 1, ...: rows i .. i+NPRE-1 are in flight in
  // the NPRE register slots, and a slot is refilled with row i+NPRE as soon as
  // row i is unpacked.  `base` (and so the trip count) is uniform across the
  // wave, so the 16-lane shuffles stay converged.
  static_assert(NPRE == 2, "two register slots");
  // steps of this wave (uniform: the wave's first position is c0 + 4 wid)
  const int wfirst = c0 + wid * 4;
  const int nsteps = (wfirst < c1) ? (c1 - wfirst + STEP - 1) / STEP : 0;
  auto step = [&](int i, RawKV<KV, DP>& sk, RawKV<KV, DP>& sv) {
    const int u = ufirst + STEP * i;
    // The slot is always unpacked and always refilled (past the chunk's end
    // the address is clamped to its last row), the new token's row (not in the
    // cache yet) replaces it from LDS under a wave-uniform test, and the two
    // slots run back to back with no exit between them: a load that some
    // lanes or paths might skip, or registers some lanes might not read, make
    // the compiler wait for the other slot's loads too, which takes away the
    // overlap of the two slots.
    float k[DP], v[DP];
    sk.get(k);
    sv.get(v);
    if (__ballot(u == u_new) != 0) {
      const bool mine = (u == u_new);
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        k[e] = mine ? knew[li * DP + e] : k[e];
        v[e] = mine ? vnew[li * DP + e] : v[e];
      }
    }
    const int un = min(u + STEP * NPRE, c1 - 1);
    sk.load(kb + (size_t)un * D + li * DP);
    sv.load(vb + (size_t)un * D + li * DP);
    fold(u, k, v);
  };
  int i = 0;
  for (; i + 1 < nsteps; i += 2) {
    step(i, pk[0], pv[0]);
    step(i + 1, pk[1], pv[1]);
  }
  if (i < nsteps) step(i, pk[0], pv[0]);
  st.template merge_xor<16>();
  st.template merge_xor<32>();
  if (lane < 16) {
#pragma unroll
    for (int r = 0; r < REP; ++r) {
      if (lane == 0) { sm[wid][r] = st.m[r]; sl[wid][r] = st.l[r]; }
#pragma unroll
      for (int e = 0; e < DP; ++e) so[wid][r][li * DP + e] = st.o[r][e];
    }
  }
  __syncthreads();

  for (int idx = tid; idx < REP * D; idx += 64 * NW) {
    const int r = idx / D, e = idx % D;
    float M = sm[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w][r]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = (sm[w][r] == -INFINITY) ? 0.f : exp2f(sm[w][r] - M);
      L += sl[w][r] * a;
      O += so[w][r][e] * a;
    }
    const int h = j * REP + r;
    if constexpr (ONE) {
      // position 0 is always attended, so L > 0
      const size_t o = ((size_t)b * p.nq + h) * D + e;
      if (p.o_dt == DT_BF16) reinterpret_cast<bf16*>(p.out)[o] = (bf16)(O / L);
      else reinterpret_cast<float*>(p.out)[o] = O / L;
    } else {
      float* pr = p.part + (((size_t)b * p.nq + h) * p.nchunks + c) * (D + 2);
      pr[e] = O;
      if (e == 0) { pr[D] = M; pr[D + 1] = L; }
    }
  }
}

// Combines the chunk partials of each (sequence, query head): one wave per
// pair.  Every load of the first 32 chunks is issued at once (the chunk
// maxima and sums by lane, the output slices for each lane's d/64 elements),
// so a short context costs a single memory round trip; longer contexts loop.
template <typename TO, int D>
__global__ __launch_bounds__(64) void attn_combine_kernel(const float* __restrict__ part,
                                                          const int32_t* __restrict__ positions, int nq,
                                                          int chunk, int nchunks, TO* __restrict__ out,
                                                          const float* __restrict__ gate, int ldg) {
  constexpr int ST = D + 2, NE = D / 64, CB = 32;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  // gated variant: this head's output gate (requested first, applied at the store)
  float gv[NE];
  if (gate != nullptr) {
#pragma unroll
    for (int e = 0; e < NE; ++e) gv[e] = gate[(size_t)b * ldg + (size_t)(2 * h + 1) * D + lane + 64 * e];
  }
  const float* pr = part + ((size_t)b * nq + h) * nchunks * ST;
  const int nvalid = (positions[b] + chunk) / chunk;
  float M = -INFINITY, L = 0.f, o[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) o[e] = 0.f;
  for (int c0 = 0; c0 < nvalid; c0 += CB) {
    const int n = min(CB, nvalid - c0);
    // lane c < n holds chunk c0 + c's max and sum; every lane holds its output
    // slice of each chunk.  The loads are unconditional (chunks past the
    // last re-read it and get weight 0), so they all go out together.
    const float* pl = pr + (size_t)(c0 + min(lane, n - 1)) * ST;
    const float mraw = pl[D], lraw = pl[D + 1];
    float ov[CB][NE];
#pragma unroll
    for (int i = 0; i < CB; ++i)
#pragma unroll
      for (int e = 0; e < NE; ++e) ov[i][e] = pr[(size_t)(c0 + min(i, n - 1)) * ST + lane + 64 * e];
    const float mc = (lane < n) ? mraw : -INFINITY;
    const float mb = wave_max(mc);
    const float mn = fmaxf(M, mb);
    const float corr = (M == -INFINITY) ? 0.f : exp2f(M - mn);
    const float wl = (lane < n) ? exp2f(mc - mn) : 0.f;
    L = L * corr + wave_sum((lane < n) ? lraw * wl : 0.f);
#pragma unroll
    for (int e = 0; e < NE; ++e) o[e] *= corr;
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
#pragma unroll
      for (int e = 0; e < NE; ++e) o[e] = fmaf(wi, ov[i][e], o[e]);
    }
    M = mn;
  }
  const float invL = 1.f / L;
  TO* orow = out + ((size_t)b * nq + h) * D;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    float y = o[e] * invL;
    if (gate != nullptr) y = y / (1.f + __expf(-gv[e]));
    orow[lane + 64 * e] = from_f32<TO>(y);
  }
}

hipError_t attn_combine(const float* part, const int32_t* positions, int B, int nq, int d, int chunk,
                        int nchunks, void* out, int o_dt, hipStream_t s, const float* gate, int ldg) {
  if (B <= 0) return hipSuccess;
  const dim3 grid(nq, B);
  if (d == 128 && o_dt == DT_BF16)
    attn_combine_kernel<bf16, 128><<<grid, 64, 0, s>>>(part, positions, nq, chunk, nchunks, (bf16*)out, gate, ldg);
  else if (d == 128)
    attn_combine_kernel<float, 128><<<grid, 64, 0, s>>>(part, positions, nq, chunk, nchunks, (float*)out, gate, ldg);
  else if (d == 256 && o_dt == DT_BF16)
    attn_combine_kernel<bf16, 256><<<grid, 64, 0, s>>>(part, positions, nq, chunk, nchunks, (bf16*)out, gate, ldg);
  else if (d == 256)
    attn_combine_kernel<float, 256><<<grid, 64, 0, s>>>(part, positions, nq, chunk, nchunks, (float*)out, gate, ldg);
  else if (d == 64 && o_dt == DT_BF16)
    attn_combine_kernel<bf16, 64><<<grid, 64, 0, s>>>(part, positions, nq, chunk, nchunks, (bf16*)out, gate, ldg);
  else if (d == 64)
    attn_combine_kernel<float, 64><<<grid, 64, 0, s>>>(part, positions, nq, chunk, nchunks, (float*)out, gate, ldg);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename KV, int D, int REP>
static void decode_launch(const AttnDecodeParams& p, hipStream_t s) {
  if constexpr (REP * D <= ATTN_ONEPASS_MAX_REP_D) {
    if (p.out != nullptr) {
      attn_decode_kernel<KV, D, REP, true><<<dim3(1, p.nkv, p.B), 1024, 0, s>>>(p);
      return;
    }
  }
  attn_decode_kernel<KV, D, REP, false><<<dim3(p.nchunks, p.nkv, p.B), 256, 0, s>>>(p);
}

template <typename KV, int D>
static hipError_t decode_rep(const AttnDecodeParams& p, hipStream_t s) {
  switch (p.nq / p.nkv) {
    case 1: decode_launch<KV, D, 1>(p, s); break;
    case 2: decode_launch<KV, D, 2>(p, s); break;
    case 4: decode_launch<KV, D, 4>(p, s); break;
    case 8: decode_launch<KV, D, 8>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool attn_decode_onepass_ok(int nq, int nkv, int d) {
  if (nkv <= 0 || nq % nkv != 0) return false;
  const int rep = nq / nkv;
  return (rep == 1 || rep == 2 || rep == 4 || rep == 8) && (d == 64 || d == 128 || d == 256) &&
         rep * d <= ATTN_ONEPASS_MAX_REP_D;
}

hipError_t attn_decode(const AttnDecodeParams& p, hipStream_t s) {
  if (p.B <= 0) return hipSuccess;
  if (p.out != nullptr && !attn_decode_onepass_ok(p.nq, p.nkv, p.d)) return hipErrorInvalidValue;
  if (p.kv_dt == DT_BF16) {
    if (p.d == 128) return decode_rep<bf16, 128>(p, s);
    if (p.d == 64) return decode_rep<bf16, 64>(p, s);
    if (p.d == 256) return decode_rep<bf16, 256>(p, s);
  } else {
    if (p.d == 128) return decode_rep<float, 128>(p, s);
    if (p.d == 64) return decode_rep<float, 64>(p, s);
    if (p.d == 256) return decode_rep<float, 256>(p, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ prefill (vector path)
// One wave per (query, head); four queries of one head per workgroup.
template <typename TQ, typename KV, int D, typename TO>
__global__ __launch_bounds__(256) void attn_prefill_vec_kernel(const AttnPrefillParams p) {
  constexpr int DP = D / 16;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int grp = lane >> 4, li = lane & 15;
  const int t = blockIdx.x * 4 + wid;
  const int h = blockIdx.y, b = blockIdx.z;
  if (t >= p.S) return;
  const int rep = p.nq / p.nkv;
  const int j = h / rep;
  const int slot = p.slots[b];
  const size_t kvoff = (size_t)slot * p.slot_stride + (size_t)j * p.head_stride;
  const KV* kb = reinterpret_cast<const KV*>(p.kcache) + kvoff;
  const KV* vb = reinterpret_cast<const KV*>(p.vcache) + kvoff;
  const size_t qrow = ((size_t)b * p.S + t) * p.nq * D + h * D;
  const TQ* qp = reinterpret_cast<const TQ*>(p.q) + qrow;
  float q[1][DP];
  const float qscale = p.scale * LOG2E;
#pragma unroll
  for (int e = 0; e < DP; ++e) q[0][e] = to_f32(qp[li * DP + e]) * qscale;
  SoftState<1, DP> st;
  st.init();
  attend<KV, D, 1>(st, q, kb, vb, 0, t + 1, 4, grp, li, -1, nullptr, nullptr);
  st.template merge_xor<16>();
  st.template merge_xor<32>();
  if (lane < 16) {
    TO* o = reinterpret_cast<TO*>(p.out) + qrow;
    const float inv = 1.f / st.l[0];
#pragma unroll
    for (int e = 0; e < DP; ++e) o[li * DP + e] = from_f32<TO>(st.o[0][e] * inv);
  }
}

template <typename TQ, typename KV, typename TO>
static hipError_t prefill_vec(const AttnPrefillParams& p, hipStream_t s) {
  const dim3 grid((p.S + 3) / 4, p.nq, p.B);
  if (p.d == 128)
    attn_prefill_vec_kernel<TQ, KV, 128, TO><<<grid, 256, 0, s>>>(p);
  else if (p.d == 64)
    attn_prefill_vec_kernel<TQ, KV, 64, TO><<<grid, 256, 0, s>>>(p);
  else if (p.d == 256)
    attn_prefill_vec_kernel<TQ, KV, 256, TO><<<grid, 256, 0, s>>>(p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t attn_prefill_vec(const AttnPrefillParams& p, hipStream_t s) {
  if (p.B <= 0 || p.S <= 0) return hipSuccess;
  if (p.kv_dt == DT_BF16) {
    if (p.q_dt == DT_BF16 && p.o_dt == DT_BF16) return prefill_vec<bf16, bf16, bf16>(p, s);
    if (p.q_dt == DT_F32 && p.o_dt == DT_F32) return prefill_vec<float, bf16, float>(p, s);
  } else if (p.q_dt == DT_F32 && p.o_dt == DT_F32) {
    return prefill_vec<float, float, float>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fsk
