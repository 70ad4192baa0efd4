// Bandwidth-bound GEMV for the decode path and other calls with few rows
// (kernel templates and launchers; gemv.hip and gemv_f8.hip instantiate them).
//
// y[m, n] = sum_k W[n, k] * a[m, k], with W stored [out, in] ("Coming back to
// Failed Star", First sitting, item 3).  Each wave streams RPW weight rows
// with 16-byte loads, lane l covering the 8-element chunks l, l+64, l+128, ...
// of every row, so the 64 lanes of a wave together span the whole reduction
// length: the RMSNorm of the activation row (fused prologue) is one wave sum,
// with no LDS staging or workgroup barrier.  Loads complete in order and the
// compiler waits for every load before the one a use needs, so the order of
// requests is the design: the one-row path requests the residual values it
// will add to, then the activation row and norm weight, then the weights (the
// norm runs while the weights are in flight); every load is unconditional
// (clamped addresses); the lm_head's next row group is in flight while the
// current one is reduced.  Cross-lane sums run on DPP row operations.
// Epilogues: plain store, residual add, SwiGLU on paired gate/up rows, and
// lm_head logits with a per-workgroup argmax (reduced by argmax_partials).
// Int8 and fp8 (e4m3) weights (one scale per row) stream 16 codes per lane
// per load; each row's dot product is multiplied by its scale before the
// epilogue.  With fp8 weights the RMSNorm-fused inputs (Q/K/V, gate/up, head)
// are quantized too, per activation row in the prologue: scale = the smallest
// power of two >= max|row| / 448, values rounded to the nearest e4m3 code
// (the hardware conversion, which rounds as the library's quantizer does:
// ties to even), the row's scale applied with the weight's in the epilogue.
#pragma once
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace fsk {

static constexpr int GEMV_THREADS = 256;
static constexpr int GEMV_WAVES = 4;
static constexpr int GEMV_LOGITS_GROUPS = 4;   // row groups per wave for the lm_head (measured: 2, 8, 16 slower)

// One lane's chunk of a weight row: CE consecutive elements.
template <typename W> struct Raw;
template <> struct Raw<bf16> { static constexpr int CE = 8; u32x4 v; };
template <> struct Raw<float> { static constexpr int CE = 8; f32x4 a, b; };
template <> struct Raw<int8_t> { static constexpr int CE = 16; u32x4 v; };
struct f8 { uint8_t c; };     // tag of e4m3 weight codes
template <> struct Raw<f8> { static constexpr int CE = 16; u32x4 v; };

__device__ __forceinline__ void raw_load(const bf16* p, Raw<bf16>& r) {
  r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void raw_load(const float* p, Raw<float>& r) {
  r.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  r.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
}
__device__ __forceinline__ void raw_load(const int8_t* p, Raw<int8_t>& r) {
  r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void raw_load(const f8* p, Raw<f8>& r) {
  r.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void raw_zero(Raw<f8>& r) { r.v = u32x4{0, 0, 0, 0}; }
// e4m3 codes to fp32 with the hardware conversion, two codes per instruction
// (exact; the library's codes are never the NaN pattern)
__device__ __forceinline__ void raw_f32(const Raw<f8>& r, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.v[i], false);   // bytes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.v[i], true);    // bytes 2, 3
    o[4 * i] = lo[0]; o[4 * i + 1] = lo[1]; o[4 * i + 2] = hi[0]; o[4 * i + 3] = hi[1];
  }
}
__device__ __forceinline__ void raw_zero(Raw<int8_t>& r) { r.v = u32x4{0, 0, 0, 0}; }
__device__ __forceinline__ void raw_zero(Raw<bf16>& r) { r.v = u32x4{0, 0, 0, 0}; }
__device__ __forceinline__ void raw_zero(Raw<float>& r) { r.a = f32x4{0, 0, 0, 0}; r.b = r.a; }
__device__ __forceinline__ void raw_f32(const Raw<bf16>& r, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(r.v[i] << 16);
    o[2 * i + 1] = __uint_as_float(r.v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void raw_f32(const Raw<int8_t>& r, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) codes4(r.v[i], o + 4 * i);
}
// CE consecutive activations (fp32)
template <int CE>
__device__ __forceinline__ void load_act(const float* p, float* o) {
#pragma unroll
  for (int h = 0; h < CE / 8; ++h) load8(p + 8 * h, o + 8 * h);
}
__device__ __forceinline__ void raw_f32(const Raw<float>& r, float* o) {
  o[0] = r.a[0]; o[1] = r.a[1]; o[2] = r.a[2]; o[3] = r.a[3];
  o[4] = r.b[0]; o[5] = r.b[1]; o[6] = r.b[2]; o[7] = r.b[3];
}

// Weight row for the i-th row slot of a wave.  SWIGLU: "rows" walk features,
// even slots read the gate row and odd slots the up row of the packed matrix.
template <int EPI>
__device__ __forceinline__ int weight_row(int slot_row, int& feature) {
  if (EPI == EPI_SWIGLU) {
    feature = slot_row >> 1;
    return ((feature >> 5) << 6) + (feature & 31) + ((slot_row & 1) << 5);
  }
  feature = slot_row;
  return slot_row;
}

template <typename W, int EPI, int MB, int CPL, int RPW, bool AQ = false>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_kernel(const GemvParams p) {
  constexpr int CE = Raw<W>::CE;
  constexpr bool QUANT = (CE == 16);
  // activations held in registers when they fit (always for one row)
  constexpr bool XREG = (MB * CPL * CE <= 64);
  const int K = p.K;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m0 = blockIdx.y * MB;
  const int mcount = min(MB, p.M - m0);
  const W* __restrict__ w = reinterpret_cast<const W*>(p.w);
  const int nchunk = K / CE;
  const int slots_total = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;   // weight rows to cover
  constexpr int GROUPS = (EPI == EPI_LOGITS) ? GEMV_LOGITS_GROUPS : 1;
  const int rows_per_block = GEMV_WAVES * RPW * GROUPS;

  // Weight loads are unconditional: past a row's end a lane re-reads the
  // row's last chunk and past the last row a wave re-reads that row (both
  // ignored below).  A load that some lanes skip makes the compiler wait for
  // every earlier load at each use, which serialises the row groups.
  auto load_group = [&](int g, Raw<W> (&raw)[CPL][RPW]) {
    const int rbase = blockIdx.x * rows_per_block + (g * GEMV_WAVES + wid) * RPW;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(lane + 64 * j, nchunk - 1);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        int f;
        const int r = weight_row<EPI>(min(rbase + i, slots_total - 1), f);
        raw_load(w + (size_t)r * K + c * CE, raw[j][i]);
      }
    }
  };
  Raw<W> ra[CPL][RPW], rb[CPL][RPW];
  // RESID: the residual values this wave adds to are requested first (each
  // output element belongs to one wave), so the epilogue needs no further
  // round trip
  float old[EPI == EPI_RESID ? RPW : 1][MB];
  if constexpr (EPI == EPI_RESID) {
    static_assert(GROUPS == 1, "one row group per wave");
    const int rb0 = blockIdx.x * rows_per_block + wid * RPW;
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int m = 0; m < MB; ++m)
        old[i][m] = p.out[(size_t)(m0 + min(m, mcount - 1)) * p.ldo + min(rb0 + i, slots_total - 1)];
  }
  static_assert(!AQ || XREG, "activation quantization keeps the rows in registers");
  float inv[MB];
  float asc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) asc[m] = 1.f;
  float xv[XREG ? MB : 1][XREG ? CPL : 1][CE];
  if constexpr (XREG) {
    // the activation rows and the norm weight are requested before the
    // weights (the counter of outstanding loads is in order), so the RMSNorm
    // runs while the weights are in flight
    float gm[CPL][CE];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      const int cc = min(c, nchunk - 1);
#pragma unroll
      for (int m = 0; m < MB; ++m)
        load_act<CE>(p.a + (size_t)(m0 + min(m, mcount - 1)) * p.lda + cc * CE, xv[m][j]);
      if (p.gamma != nullptr) load_act<CE>(p.gamma + cc * CE, gm[j]);
    }
    load_group(0, ra);
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      if (lane + 64 * j >= nchunk) {      // past the row's end: zero activations
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int e = 0; e < CE; ++e) xv[m][j][e] = 0.f;
      }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < CE; ++e) ss = fmaf(xv[m][j][e], xv[m][j][e], ss);
      inv[m] = (p.gamma != nullptr) ? rsqrtf(wave_sum(ss) / (float)K + p.eps) : 1.f;
    }
    if (p.gamma != nullptr) {
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int e = 0; e < CE; ++e) xv[m][j][e] *= inv[m] * gm[j][e];
    }
    if constexpr (AQ) {
      // the fp8 activation rule on each normalised row: codes kept as their values, scale in asc
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int e = 0; e < CE; ++e) amax = fmaxf(amax, fabsf(xv[m][j][e]));
        const float sc = f8_row_scale(wave_max(amax));
        asc[m] = sc;
        // x / sc: a power-of-two scale of at least 2^-126 has an exact fp32
        // reciprocal; below it (rows of magnitude under ~2^-117) divide
        const bool recip = sc >= 1.17549435e-38f;
        const float isc = recip ? 1.f / sc : 0.f;
        // round to e4m3 and back with the hardware conversions (round to
        // nearest even; |x / sc| <= 448, so nothing saturates; a negative
        // value that rounds to zero becomes -0, the same value)
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int e = 0; e < CE; e += 2) {
            float q0 = recip ? xv[m][j][e] * isc : (sc > 0.f ? xv[m][j][e] / sc : 0.f);
            float q1 = recip ? xv[m][j][e + 1] * isc : (sc > 0.f ? xv[m][j][e + 1] / sc : 0.f);
            const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
            const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
            xv[m][j][e] = d[0];
            xv[m][j][e + 1] = d[1];
          }
      }
    }
  } else {
    load_group(0, ra);          // weights first: their latency covers the prologue
    // ---- prologue: per-row RMSNorm scale from this wave's own slices
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const float* arow = p.a + (size_t)(m0 + min(m, mcount - 1)) * p.lda;
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        float v[CE];
        if (c < nchunk) load_act<CE>(arow + c * CE, v);
        else {
#pragma unroll
          for (int e = 0; e < CE; ++e) v[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < CE; ++e) ss = fmaf(v[e], v[e], ss);
      }
      inv[m] = (p.gamma != nullptr) ? rsqrtf(wave_sum(ss) / (float)K + p.eps) : 1.f;
    }
  }

  float best_v[MB];
  int best_i[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) { best_v[m] = 0.f; best_i[m] = -1; }

  auto compute = [&](int g, const Raw<W> (&raw)[CPL][RPW]) {
    const int rbase = blockIdx.x * rows_per_block + (g * GEMV_WAVES + wid) * RPW;
    if (rbase >= slots_total) return;
    float acc[RPW][MB];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[i][m] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c >= nchunk) continue;
      float gam[CE];
      if (!XREG) {
        if (p.gamma != nullptr) load_act<CE>(p.gamma + c * CE, gam);
        else {
#pragma unroll
          for (int e = 0; e < CE; ++e) gam[e] = 1.f;
        }
      }
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        float a[CE];
        if (XREG) {
#pragma unroll
          for (int e = 0; e < CE; ++e) a[e] = xv[XREG ? m : 0][XREG ? j : 0][e];
        } else {
          load_act<CE>(p.a + (size_t)(m0 + min(m, mcount - 1)) * p.lda + c * CE, a);
#pragma unroll
          for (int e = 0; e < CE; ++e) a[e] *= inv[m] * gam[e];
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          float wv[CE];
          raw_f32(raw[j][i], wv);
          float s = acc[i][m];
#pragma unroll
          for (int e = 0; e < CE; ++e) s = fmaf(wv[e], a[e], s);
          acc[i][m] = s;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[i][m] = wave_sum(acc[i][m]);

    // ---- epilogue (every lane holds the sums; lane 0 writes)
    if (lane == 0) {
      if (QUANT) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          int f;
          const int r = weight_row<EPI>(min(rbase + i, slots_total - 1), f);
          const float sc = p.wscale[r];
#pragma unroll
          for (int m = 0; m < MB; ++m) acc[i][m] *= AQ ? sc * asc[m] : sc;
        }
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int sr = rbase + i;
        if (sr >= slots_total) continue;
        int f;
        weight_row<EPI>(sr, f);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m >= mcount) continue;
          const size_t o = (size_t)(m0 + m) * p.ldo + f;
          if (EPI == EPI_STORE) {
            p.out[o] = acc[i][m];
          } else if (EPI == EPI_RESID) {
            p.out[o] = old[EPI == EPI_RESID ? i : 0][m] + acc[i][m];
          } else if (EPI == EPI_SWIGLU) {
            // slot rows come in (gate, up) pairs: i even = gate, i + 1 = up
            if ((i & 1) == 0) p.out[o] = silu(acc[i][m]) * acc[(i + 1) % RPW][m];
          } else {  // EPI_LOGITS
            const float v = acc[i][m];
            if (p.logits) p.logits[o] = v;
            if (__builtin_isfinite(v) && better(v, f, best_v[m], best_i[m])) { best_v[m] = v; best_i[m] = f; }
          }
        }
      }
    }
  };

  // ping-pong over row groups with statically indexed register buffers: group
  // g + 1 is in flight while group g is reduced (no load is conditional, and
  // the last pair is peeled off the rolled loop)
  if constexpr (GROUPS == 1) {
    compute(0, ra);
  } else {
    static_assert(GROUPS % 2 == 0, "row groups come in pairs");
#pragma unroll 1
    for (int g = 0; g < GROUPS - 2; g += 2) {
      load_group(g + 1, rb);
      compute(g, ra);
      load_group(g + 2, ra);
      compute(g + 1, rb);
    }
    load_group(GROUPS - 1, rb);
    compute(GROUPS - 2, ra);
    compute(GROUPS - 1, rb);
  }

  if (EPI == EPI_LOGITS) {
    // block-level best per row; argmax_partials reduces the blocks afterwards
    __shared__ float bvs[GEMV_WAVES][MB];
    __shared__ int bis[GEMV_WAVES][MB];
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m) { bvs[wid][m] = best_v[m]; bis[wid][m] = best_i[m]; }
    }
    __syncthreads();
    if ((int)threadIdx.x < mcount) {
      const int m = threadIdx.x;
      float bv = bvs[0][m];
      int bi = bis[0][m];
      for (int ww = 1; ww < GEMV_WAVES; ++ww)
        if (better(bvs[ww][m], bis[ww][m], bv, bi)) { bv = bvs[ww][m]; bi = bis[ww][m]; }
      p.part_val[(size_t)m * gridDim.x + blockIdx.x] = bv;
      p.part_idx[(size_t)m * gridDim.x + blockIdx.x] = bi;
    }
  }
}

// ------------------------------------------------------------------ launcher
// chunks per lane for a reduction length K in chunks of ce elements
static int cpl_for(int K, int ce) {
  const int c = (K / ce + 63) / 64;
  if (c <= 1) return 1;
  if (c <= 2) return 2;
  if (c <= 4) return 4;
  if (c <= 6) return 6;
  if (c <= 8) return 8;
  return -1;
}

// Rows per wave.  The decode projections run fastest at a few hundred
// workgroups with a few KB of weights per wave (measured per class): SwiGLU
// takes rows in (gate, up) pairs; one-row calls with at least 2048 output
// rows (QKV) and SwiGLU two bf16 / fp32 rows or four int8 rows per wave;
// smaller one-row calls (O, down) one row; the lm_head one bf16 / fp32 row or
// four int8 rows per wave over its row groups; several activation rows two
// (int8: four for one-chunk rows).
static constexpr int logits_rpw(bool quant) { return quant ? 4 : 1; }
static int rpw_for(int epi, bool quant, int M, int cpl, int slots) {
  if (epi == EPI_LOGITS) return logits_rpw(quant);
  if (M > 1) return quant ? (cpl <= 1 ? 4 : 2) : 2;
  if (epi == EPI_SWIGLU || slots >= 2048) return quant ? 4 : 2;
  return 1;
}


template <typename W, int EPI, int MB, int CPL, int RPW>
static hipError_t launch_rpw(GemvParams p, hipStream_t s) {
  constexpr bool XR = (MB * CPL * Raw<W>::CE <= 64);
  const int slots_total = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const int rows_per_group = GEMV_WAVES * RPW;
  const int groups = (EPI == EPI_LOGITS) ? GEMV_LOGITS_GROUPS : 1;
  const int gx = (slots_total + rows_per_group * groups - 1) / (rows_per_group * groups);
  p.groups = groups;
  const int gy = (p.M + MB - 1) / MB;
  if constexpr (std::is_same<W, f8>::value && EPI != EPI_RESID) {
    // fp8 weights: the RMSNorm-fused inputs are always quantized (rows in registers)
    if (!p.aquant) return hipErrorInvalidValue;
    if constexpr (XR) {
      gemv_kernel<W, EPI, MB, CPL, RPW, true><<<dim3(gx, gy), GEMV_THREADS, 0, s>>>(p);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    if (p.aquant) return hipErrorInvalidValue;
    gemv_kernel<W, EPI, MB, CPL, RPW><<<dim3(gx, gy), GEMV_THREADS, 0, s>>>(p);
    return hipGetLastError();
  }
}

template <typename W, int EPI, int MB, int CPL>
static hipError_t launch_gemv(GemvParams p, hipStream_t s) {
  constexpr bool QUANT = Raw<W>::CE == 16;
  const int slots = (EPI == EPI_SWIGLU) ? 2 * p.N : p.N;
  const int r = rpw_for(EPI, QUANT, p.M, CPL, slots);
  // the instantiations each kind of call can reach
  if constexpr (EPI == EPI_LOGITS) {
    return launch_rpw<W, EPI, MB, CPL, logits_rpw(QUANT)>(p, s);
  } else {
    if constexpr (MB == 1 && EPI != EPI_SWIGLU) {
      if (r == 1) return launch_rpw<W, EPI, MB, CPL, 1>(p, s);
    }
    if constexpr (QUANT) {
      if (r == 4) return launch_rpw<W, EPI, MB, CPL, 4>(p, s);
    }
    if (r == 2) return launch_rpw<W, EPI, MB, CPL, 2>(p, s);
    return hipErrorInvalidValue;
  }
}

template <typename W, int EPI, int MB>
static hipError_t dispatch_cpl(GemvParams p, hipStream_t s) {
  if constexpr (Raw<W>::CE == 16) {
    // 16 codes per chunk: K <= 4096 needs at most 4 chunks per lane
    switch (cpl_for(p.K, 16)) {
      case 1: return launch_gemv<W, EPI, MB, 1>(p, s);
      case 2: return launch_gemv<W, EPI, MB, 2>(p, s);
      case 4: return launch_gemv<W, EPI, MB, 4>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (cpl_for(p.K, Raw<W>::CE)) {
    case 1: return launch_gemv<W, EPI, MB, 1>(p, s);
    case 2: return launch_gemv<W, EPI, MB, 2>(p, s);
    case 4: return launch_gemv<W, EPI, MB, 4>(p, s);
    case 6: return launch_gemv<W, EPI, MB, 6>(p, s);
    case 8: return launch_gemv<W, EPI, MB, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Rows per workgroup: 1, 4, or 8 (5-8 rows and larger M in groups of 8), so a
// short prompt streams each weight once.
template <typename W, int EPI>
static hipError_t dispatch_mb(GemvParams p, hipStream_t s) {
  if (p.M == 1) return dispatch_cpl<W, EPI, 1>(p, s);
  if (EPI == EPI_LOGITS) {
    if (p.M > GEMV_LOGITS_MAX_M) return hipErrorInvalidValue;
    return dispatch_cpl<W, EPI, 4>(p, s);
  } else {
    if (p.M <= 4) return dispatch_cpl<W, EPI, 4>(p, s);
    return dispatch_cpl<W, EPI, 8>(p, s);
  }
}

}  // namespace fsk
