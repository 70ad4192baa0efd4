// Seeded sampling of a logits row: temperature -> top-k -> top-p ->
// renormalise -> draw ("Coming back to Failed Star", section "Next: one
// complete deterministic generation arc": the sampling arc with an explicit
// filter order; "ferrite", What it does: temperature, top-k, top-p).
//
// Rules (the pages fix only the order): finite logits only; top-k keeps every
// logit >= the k-th largest (ties at the cut all kept, k = 0 no limit); top-p
// keeps every token at least as probable as the one at which the ranked
// cumulative mass of the top-k set first reaches p; the kept probabilities are
// renormalised and the caller's uniform u is mapped through their cumulative
// distribution in increasing token ID.
//
// No sort.  Logits map to order-preserving 32-bit keys; the top-k cut is the
// k-th largest key, found by a three-level radix select (12 + 12 + 8 bits) on
// count histograms; the top-p cut is the largest key whose tail mass reaches
// p * Z_k, found the same way on histograms of probability mass
// 2^((x - max) log2(e) / T).  The draw sums the kept mass per block of token
// IDs, then one workgroup walks the block sums and the chosen block's IDs.
// Every pass is one launch over (blocks of IDs) x (rows).  A pass first makes
// the one selection that the previous pass's histogram allows (every block
// makes it identically, from the same global histogram in a fixed order;
// block 0 stores it in the row scratch), then builds the next histogram, so
// no separate selection step runs between launches and no pass repeats an
// earlier selection.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace fsk {

namespace {

constexpr int NT = 256;      // threads per block
constexpr int PER = 8;       // IDs per thread requested together (a block's slice in one round trip)
constexpr int NB1 = 4096;    // bins, levels 1 and 2 (12 bits each)
constexpr int NB3 = 256;     // bins, level 3 (8 bits)

__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float keyf(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ bool finite(float f) { return (__float_as_uint(f) & 0x7f800000u) != 0x7f800000u; }

// Inclusive prefix over the NT threads of a block: a wave64 shuffle scan, then
// the four wave totals folded in a fixed order, so every block computes
// bit-identical results.  Returns this thread's inclusive sum; *before
// receives the previous thread's inclusive sum (0 for thread 0) and *total the
// block total, so neighbouring intervals [before, inclusive] meet exactly.
template <typename T>
__device__ T block_inclusive(T v, T* before, T* total) {
  static_assert(NT == 256, "four waves");
  __shared__ T ws[NT / 64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  T x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) ws[w] = x;
  __syncthreads();
  T off = T(0);
  for (int i = 0; i < w; ++i) off += ws[i];
  T tot = T(0);
  for (int i = 0; i < NT / 64; ++i) tot += ws[i];
  const T inc = x + off;
  const T prev = __shfl_up(inc, 1);
  *before = lane > 0 ? prev : off;
  *total = tot;
  __syncthreads();
  return inc;
}

// Descending-order selection over a histogram of nb bins (count or mass):
// the bin b where the bins above b hold < target and b brings the total to
// >= target, and target minus what lies above.  When rounding leaves the
// total short of target, the lowest non-empty bin.  Called by all NT threads;
// every thread gets the result.
template <typename T, int NB>
__device__ void select_desc(const T* h, T target, int* out_bin, T* out_rem) {
  static_assert(NB % NT == 0, "whole bins per thread");
  constexpr int W = NB / NT;                  // bins per thread (16 or 1)
  __shared__ int sbin;
  __shared__ T srem;
  const int t = threadIdx.x;
  const int hi = NB - t * W;                  // thread t owns bins [hi - W, hi), read downward
  T hv[W];                                    // all of them requested at once, kept for the walk
#pragma unroll
  for (int i = 0; i < W; ++i) hv[i] = h[hi - 1 - i];
  T s = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) s += hv[i];
  if (t == 0) sbin = -1;
  __syncthreads();
  T above, total;
  const T upto = block_inclusive<T>(s, &above, &total);
  if (above < target && upto >= target) {     // exactly one thread's interval holds target
    // descending walk: the first non-empty bin that brings the mass to target
    // (or, failing that, the last non-empty bin seen)
    T a = above, last_a = above;
    int last = -1;
    bool done = false;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if (!done) {
        const T v = hv[i];
        if (v > 0) {
          last = hi - 1 - i;
          last_a = a;
          done = (a + v >= target);
        }
        a += v;
      }
    }
    if (last >= 0) { sbin = last; srem = target - last_a; }
  }
  __syncthreads();
  if (sbin < 0 && t == 0) {                   // total fell short: lowest non-empty bin
    int b = 0;
    for (int i = 0; i < NB; ++i) if (h[i] > 0) { b = i; break; }
    sbin = b;
    srem = h[b];
  }
  __syncthreads();
  *out_bin = sbin;
  *out_rem = srem;
  __syncthreads();
}

// Sum of a histogram in a fixed order (identical in every block)
template <typename T, int NB>
__device__ T hist_total(const T* h) {
  constexpr int W = NB / NT;
  T hv[W];
#pragma unroll
  for (int i = 0; i < W; ++i) hv[i] = h[threadIdx.x * W + i];
  T s = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) s += hv[i];
  T before, total;
  block_inclusive<T>(s, &before, &total);
  return total;
}

}  // namespace

// Clears the row scratch: blockIdx.y = row, blockIdx.x = one of ZB pieces.
constexpr int ZB = 16;
__global__ __launch_bounds__(NT) void sample_zero_kernel(SampleRowScratch* scr) {
  SampleRowScratch* sc = scr + blockIdx.y;
  uint32_t* p = reinterpret_cast<uint32_t*>(sc);
  const int n = (int)(sizeof(SampleRowScratch) / 4);
  for (int i = blockIdx.x * NT + threadIdx.x; i < n; i += ZB * NT) p[i] = 0u;
}

// mode 0: level-1 count histogram (+ max key, finite count)
// mode 1: select the top-k level-1 digit; level-2 count histogram
// mode 2: select the level-2 digit; level-3 count histogram
// mode 3: select the level-3 digit (top-k cut); level-1 mass histogram over keys >= it
// mode 4: select the top-p level-1 digit; level-2 mass histogram
// mode 5: select the level-2 digit; level-3 mass histogram
// mode 6: the final cut (top-p level 3, or the top-k cut); kept mass of this block
template <int MODE>
__global__ __launch_bounds__(NT) void sample_pass_kernel(const SampleParams p) {
  const int row = blockIdx.y;
  SampleRowScratch* sc = p.scr + row;
  const float* x = p.logits + (size_t)row * p.ld;
  const int i0 = blockIdx.x * p.slice, i1 = min(i0 + p.slice, p.V);
  // the first stretch of this block's logits is requested before anything
  // else: it does not depend on the selection below, which then runs while
  // the values are in flight (past the slice the last ID is re-read and skipped)
  float vals0[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) vals0[j] = x[min(i0 + (int)threadIdx.x + j * NT, i1 - 1)];
  if (MODE > 0 && sc->nfinite == 0) return;
  constexpr bool MASS = MODE >= 3 && MODE <= 5;
  constexpr int NB = (MODE == 2 || MODE == 5) ? NB3 : NB1;
  __shared__ uint32_t hc[NB1];
  __shared__ float hm[NB1];
  __shared__ uint32_t smax, scount;
  __shared__ float ssum;
  const bool store = blockIdx.x == 0 && threadIdx.x == 0;

  // ---- this pass's selection (earlier ones come from the scratch)
  uint32_t pre = 0, kcut = 0, cut = 0;
  int pshift = 0;
  float xmax = 0.f;
  if (MODE == 1) {
    const uint32_t nf = sc->nfinite;
    const uint32_t k = (p.top_k <= 0 || (uint32_t)p.top_k > nf) ? nf : (uint32_t)p.top_k;
    int b;
    uint32_t r;
    select_desc<uint32_t, NB1>(sc->c1, k, &b, &r);
    if (store) { sc->kb1 = (uint32_t)b; sc->kr1 = r; }
    pre = (uint32_t)b;
    pshift = 20;
  } else if (MODE == 2) {
    int b;
    uint32_t r;
    const uint32_t b1 = sc->kb1;
    select_desc<uint32_t, NB1>(sc->c2, sc->kr1, &b, &r);
    if (store) { sc->kb2 = (uint32_t)b; sc->kr2 = r; }
    pre = (b1 << 12) | (uint32_t)b;
    pshift = 8;
  } else if (MODE == 3) {
    if (p.top_k > 0) {
      int b;
      uint32_t r;
      select_desc<uint32_t, NB3>(sc->c3, sc->kr2, &b, &r);
      kcut = (sc->kb1 << 20) | (sc->kb2 << 8) | (uint32_t)b;
    } else {
      kcut = 0u;                              // no top-k: every finite key is kept
    }
    if (store) sc->kcut = kcut;
  } else if (MODE == 4) {
    const float z = hist_total<float, NB1>(sc->m1);
    int b;
    float r;
    select_desc<float, NB1>(sc->m1, p.top_p * z, &b, &r);
    if (store) { sc->z = z; sc->pb1 = (uint32_t)b; sc->pr1 = r; }
    pre = (uint32_t)b;
    pshift = 20;
  } else if (MODE == 5) {
    int b;
    float r;
    const uint32_t b1 = sc->pb1;
    select_desc<float, NB1>(sc->m2, sc->pr1, &b, &r);
    if (store) { sc->pb2 = (uint32_t)b; sc->pr2 = r; }
    pre = (b1 << 12) | (uint32_t)b;
    pshift = 8;
  } else if (MODE == 6) {
    if (p.top_p < 1.f) {
      int b;
      float r;
      select_desc<float, NB3>(sc->m3, sc->pr2, &b, &r);
      cut = (sc->pb1 << 20) | (sc->pb2 << 8) | (uint32_t)b;
    } else {
      cut = sc->kcut;
    }
    if (store) sc->cut = cut;
  }
  if (MODE >= 4) kcut = sc->kcut;
  if (MODE >= 3) xmax = keyf(sc->maxkey);

  for (int b = threadIdx.x; b < NB; b += NT) { hc[b] = 0u; hm[b] = 0.f; }
  if (threadIdx.x == 0) { smax = 0u; scount = 0u; ssum = 0.f; }
  __syncthreads();
  uint32_t lmax = 0u, lcnt = 0u;
  float lsum = 0.f;
  for (int base = i0; base < i1; base += NT * PER) {
    // the thread's IDs of this stretch, all requested before any is used
    float vals[PER];
    if (base == i0) {
#pragma unroll
      for (int j = 0; j < PER; ++j) vals[j] = vals0[j];
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) vals[j] = x[min(base + (int)threadIdx.x + j * NT, i1 - 1)];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
    const int i = base + (int)threadIdx.x + j * NT;
    const float v = vals[j];
    if (i >= i1 || !finite(v)) continue;
    const uint32_t key = fkey(v);
    if (MODE == 0) {
      atomicAdd(&hc[key >> 20], 1u);
      lmax = max(lmax, key);
      ++lcnt;
    } else if (MODE == 1 || MODE == 2) {
      if ((key >> pshift) == pre) atomicAdd(&hc[MODE == 1 ? ((key >> 8) & 0xfffu) : (key & 0xffu)], 1u);
    } else {
      if (key < kcut) continue;
      const float e = __builtin_amdgcn_exp2f((v - xmax) * p.sc);
      if (MODE == 3) atomicAdd(&hm[key >> 20], e);
      else if (MODE == 4 || MODE == 5) {
        if ((key >> pshift) == pre) atomicAdd(&hm[MODE == 4 ? ((key >> 8) & 0xfffu) : (key & 0xffu)], e);
      } else if (key >= cut) {
        lsum += e;
      }
    }
    }
  }
  if (MODE == 0) {
    atomicMax(&smax, lmax);
    atomicAdd(&scount, lcnt);
  }
  if (MODE == 6) atomicAdd(&ssum, lsum);
  __syncthreads();
  if (MODE == 6) {
    if (threadIdx.x == 0) sc->bsum[blockIdx.x] = ssum;
    return;
  }
  uint32_t* gc = MODE == 0 ? sc->c1 : MODE == 1 ? sc->c2 : sc->c3;
  float* gm = MODE == 3 ? sc->m1 : MODE == 4 ? sc->m2 : sc->m3;
  for (int b = threadIdx.x; b < NB; b += NT) {
    if (MASS) { if (hm[b] != 0.f) atomicAdd(&gm[b], hm[b]); }
    else if (hc[b] != 0u) atomicAdd(&gc[b], hc[b]);
  }
  if (MODE == 0 && threadIdx.x == 0) {
    atomicMax(&sc->maxkey, smax);
    atomicAdd(&sc->nfinite, scount);
  }
}

// The interval walk shared by both levels of the draw: given this thread's
// mass v (threads in increasing token-ID order) and the target, the thread
// whose cumulative interval first exceeds target (the last thread with mass
// when rounding never lets it).  Returns that thread's index and the mass
// before it through *before; every thread gets the result.
__device__ int walk_to(float v, float target, float* before) {
  __shared__ int swho;
  __shared__ float sbefore;
  __shared__ int slast;
  if (threadIdx.x == 0) { swho = -1; slast = -1; }
  __syncthreads();
  float prev, total;
  const float inc = block_inclusive<float>(v, &prev, &total);
  if (v > 0.f) {
    if (prev <= target && inc > target) { swho = threadIdx.x; sbefore = prev; }
    atomicMax(&slast, (int)threadIdx.x);
  }
  __syncthreads();
  int who = swho;
  float bef = sbefore;
  if (who < 0) {                              // rounding: the last thread with mass
    who = max(slast, 0);
    __syncthreads();
    if ((int)threadIdx.x == who) sbefore = prev;
    __syncthreads();
    bef = sbefore;
  }
  __syncthreads();
  *before = bef;
  return who;
}

// One workgroup per row: the block of token IDs holding u * Z (a scan over
// the block sums), then the thread run holding it within that block (a scan
// over the threads' run sums), then that run's IDs in order.
__global__ __launch_bounds__(NT) void sample_final_kernel(const SampleParams p) {
  const int row = blockIdx.x;
  SampleRowScratch* sc = p.scr + row;
  if (sc->nfinite == 0) {
    if (threadIdx.x == 0) p.out[row] = -1;
    return;
  }
  static_assert(SAMPLE_MAX_BLOCKS <= NT, "one block sum per thread");
  const uint32_t cut = sc->cut;
  const float bsv = ((int)threadIdx.x < p.G) ? sc->bsum[threadIdx.x] : 0.f;
  float bprev, btot;
  block_inclusive<float>(bsv, &bprev, &btot);
  const float target = p.u[row] * btot;
  float before;
  const int blk = walk_to(bsv, target, &before);

  const float* x = p.logits + (size_t)row * p.ld;
  const float xmax = keyf(sc->maxkey);
  const int i0 = blk * p.slice, i1 = min(i0 + p.slice, p.V);
  // each thread takes a contiguous run of IDs (requested together while the
  // run fits PER; the clamped re-reads past the run are skipped)
  const int per = (p.slice + NT - 1) / NT;
  const int a0 = i0 + threadIdx.x * per, a1 = min(a0 + per, i1);
  float mine = 0.f;
  if (per <= PER) {
    float vals[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) vals[j] = x[min(a0 + j, max(a1 - 1, i0))];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const float v = vals[j];
      if (a0 + j < a1 && finite(v) && fkey(v) >= cut) mine += __builtin_amdgcn_exp2f((v - xmax) * p.sc);
    }
  } else {
    for (int i = a0; i < a1; ++i) {
      const float v = x[i];
      if (finite(v) && fkey(v) >= cut) mine += __builtin_amdgcn_exp2f((v - xmax) * p.sc);
    }
  }
  float rbefore;
  const int who = walk_to(mine, target - before, &rbefore);
  if ((int)threadIdx.x == who) {
    // the chosen run, walked by the thread that summed it (its IDs are cached)
    const float t = target - before;
    int pick = -1;
    float acc = rbefore;
    for (int i = a0; i < a1; ++i) {
      const float v = x[i];
      if (!(finite(v) && fkey(v) >= cut)) continue;
      pick = i;
      acc += __builtin_amdgcn_exp2f((v - xmax) * p.sc);
      if (acc > t) break;
    }
    p.out[row] = pick;
  }
}

// ------------------------------------------------------------------ static scratch
// Row scratch for callers that cannot allocate: one copy per device, held
// until the process ends.  Host code never passes this name to a kernel (on
// the host it only stands in for the symbol); it passes the device address
// hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) SampleRowScratch scratch[SAMPLE_STATIC_MAX_ROWS];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
SampleRowScratch* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t sample_static_scratch(SampleRowScratch** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<SampleRowScratch*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t sample_rows(const SampleParams& p, hipStream_t s) {
  if (p.B <= 0) return hipSuccess;
  if (p.G <= 0 || p.G > SAMPLE_MAX_BLOCKS) return hipErrorInvalidValue;
  const dim3 grid(p.G, p.B);
  sample_zero_kernel<<<dim3(ZB, p.B), NT, 0, s>>>(p.scr);
  sample_pass_kernel<0><<<grid, NT, 0, s>>>(p);
  if (p.top_k > 0) {                              // the top-k cut's two upper radix levels
    sample_pass_kernel<1><<<grid, NT, 0, s>>>(p);
    sample_pass_kernel<2><<<grid, NT, 0, s>>>(p);
  }
  sample_pass_kernel<3><<<grid, NT, 0, s>>>(p);   // m1: Z_k, needed by the draw too
  if (p.top_p < 1.f) {
    sample_pass_kernel<4><<<grid, NT, 0, s>>>(p);
    sample_pass_kernel<5><<<grid, NT, 0, s>>>(p);
  }
  sample_pass_kernel<6><<<grid, NT, 0, s>>>(p);
  sample_final_kernel<<<p.B, NT, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace fsk
