// C ABI of the forward pass (declared in include/fs.h): model state, argument
// validation and the order of kernel launches for prefill and decode.
//
// Forward pass ("Coming back to Failed Star", Second sitting, data-flow
// figure; "Milestones", M2): ids -> embedding -> per block [RMSNorm, QKV,
// q/k RMSNorm + RoPE, GQA attention, output projection + residual, RMSNorm,
// SwiGLU MLP + residual] -> final RMSNorm of the last row -> tied head.
// KV-cached decode ("Milestones", M4) appends one position per step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/fs.h"
#include "kernels.h"

using namespace fsk;

namespace {

thread_local std::string g_err;

fs_status fail(fs_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(FS_ERR_HIP, std::string(#expr) + " failed: " + hipGetErrorString(e_)); \
  } while (0)

// Up to this many rows per call the projections run as GEMV (weights streamed
// once, fp32 activations); above it as MFMA GEMM on bf16 activations.  With
// bf16 weights the few-row MFMA GEMM is faster from 5 rows on (the 6-token
// scorer: 1.49 -> 1.22 ms); int8 codes stay on the GEMV up to 8 rows (the GEMM
// would widen them first); with fp8 weights the GEMV quantizes its activation
// rows in registers, up to 4.
constexpr int SKINNY_MAX_ROWS = 4;
constexpr int SKINNY_MAX_ROWS_I8 = 8;
constexpr int SKINNY_MAX_ROWS_F8 = 4;
// prefill: up to this many tokens per sequence the attention runs on the
// vector kernel whatever the projections use
constexpr int ATTN_VEC_MAX_S = 32;
// fp8 weights: from this many rows a prefill's Q/K/V and gate/up products run
// on the fp8 matrix instructions (gemm_f8); below it on widened weights
constexpr int F8_GEMM_MIN_ROWS = 512;
// Few-row (<= 64) O and down projections split K over up to 12 workgroups per
// 32-column slab (N = hidden gives only hidden / 32 slabs otherwise).
constexpr int KSPLIT_MAX = 12;
static_assert(KSPLIT_MAX <= RMSNORM_MAX_PARTS, "the RMSNorm adds every partial");
constexpr int KSPLIT_MAX_ROWS = 64;
// In timing mode each call starts with a short device-side wait so the host
// can queue the whole call behind it: the event pairs then bracket kernels
// that run back to back instead of waiting on the host.
constexpr int TIMING_GATE_US = 3000;
constexpr int STAGE_RING = 64;

struct LayerW {
  void *wqkv, *wo, *wgu, *wdown;
  float *attn_norm, *q_norm, *k_norm, *mlp_norm;
  // int8 weights: one scale per weight row (null otherwise)
  float *sqkv = nullptr, *so = nullptr, *sgu = nullptr, *sdown = nullptr;
  // bf16 models: an fp8 (e4m3, power-of-two row scale) copy of the Q/K/V and
  // gate/up weights for the remainder pass of the large prefill GEMMs
  uint8_t *w8qkv = nullptr, *w8gu = nullptr;
  float *s8qkv = nullptr, *s8gu = nullptr;
  // bound on every base-2 attention score of the layer (from the q/k norm weights)
  float qk_bound = 0.f;
};

struct DecodeKey {
  int B, chunk, nchunks;
  const void *tokens, *logits, *next;
  bool operator==(const DecodeKey& o) const {
    return B == o.B && chunk == o.chunk && nchunks == o.nchunks && tokens == o.tokens &&
           logits == o.logits && next == o.next;
  }
};
struct DecodeGraph {
  DecodeKey key;
  hipGraph_t graph;
  hipGraphExec_t exec;
};
constexpr size_t MAX_GRAPHS = 32;

struct TimedLaunch {
  const char* label;
  hipEvent_t a, b;
};

template <class T>
hipError_t dalloc(T** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return hipSuccess;
  return hipMalloc(reinterpret_cast<void**>(p), bytes);
}

}  // namespace

struct fs_model {
  fs_config cfg{};
  int device = 0;
  int dt = 0;
  size_t esz = 0;
  int qkv_w = 0, qw = 0, kvw = 0;
  int qpw = 0;          // rows of the q (+ gate) projection
  int rot = 0;          // rotated dims per head
  int gated = 0;        // attention output gate carried by the q projection
  int wdt = 0;          // storage of the matrices: dt, or DT_I8 / DT_F8 (codes + row scales)
  // weights
  void* wblob = nullptr;
  size_t wblob_bytes = 0;
  float* nblob = nullptr;
  float* sblob = nullptr;         // int8 row scales
  void* wconv = nullptr;          // bf16 copy of one layer matrix's codes (MFMA operand)
  void* w8blob = nullptr;         // fp8 copies of the Q/K/V and gate/up weights (bf16 models)
  float* s8blob = nullptr;        // their row scales
  float* am_pv = nullptr;         // argmax block bests of many-row heads [max_seqs][ARGMAX_BLOCKS]
  int32_t* am_pi = nullptr;
  bool lo8 = false;               // remainder passes of the large GEMMs on fp8 operands
  void* embed = nullptr;
  float* embed_scale = nullptr;
  float* final_norm = nullptr;
  std::vector<LayerW> layers;
  // KV cache [layer][slot][kv_head][pos][d]
  void* kcache = nullptr;
  void* vcache = nullptr;
  long long head_stride = 0, slot_stride = 0, layer_stride = 0;
  float *rope_cos = nullptr, *rope_sin = nullptr;
  std::vector<int32_t> slot_len;
  // activation scratch, grown on demand
  long long scratch_rows = 0;
  float* x = nullptr;
  void* xn = nullptr;
  float* ascale = nullptr;        // fp8 option: row scales of the quantized norm outputs
  void* qkv = nullptr;
  void* qr = nullptr;
  void* attn = nullptr;
  void* hbuf = nullptr;
  // decode scratch
  int32_t* d_pos = nullptr;
  int32_t* d_slot = nullptr;      // = d_pos + max_seqs (one allocation, staged by one copy)
  float* part = nullptr;
  int max_chunks = 0;
  // split-K partials of the few-row O / down projections, [KSPLIT_MAX][64][hidden];
  // pend_np > 0: that many partials wait to be added to x by the next RMSNorm
  float* kpart = nullptr;
  int pend_np = 0;
  // where the decode attention finds this layer's q/k/v projection (m->qkv, or
  // qkv_np split-K partials in kpart)
  const float* qkv_src = nullptr;
  int qkv_np = 1;
  float* lm_pv = nullptr;
  int32_t* lm_pi = nullptr;
  float* logits_tmp = nullptr;    // [max_seqs, V] when the caller passes none
  SampleRowScratch* sample_scr = nullptr;   // [max_seqs], on the first fs_sample
  // persistent batch-1 decode step (one launch per step) where the shape allows
  bool use_persist = false;
  void* pex = nullptr;            // its exchange records
  uint32_t pstep = 0;             // steps launched (the records' tag)
  int32_t* pabort = nullptr;      // pinned host word the kernel sets when a wait times out
  int32_t* pabort_dev = nullptr;
  long long* ptrace = nullptr;    // clock stamps of the last persistent step (FS_DECODE_TRACE=1)
  // out-of-range token report: pinned host words {flag, id, row} the embedding
  // kernel writes through their device mapping (tokerr_dev)
  int32_t* tokerr = nullptr;
  int32_t* tokerr_dev = nullptr;
  int32_t* gen_tok = nullptr;     // device int32 [1]: the token fs_generate feeds back
  int32_t* gen_host = nullptr;    // pinned int32 [2]: host copies of two consecutive tokens
  hipEvent_t gen_ev[2] = {};      // their copies' completion
  // pinned staging of per-call host arrays
  int32_t* stage = nullptr;       // [STAGE_RING][2 * max_seqs]
  hipEvent_t stage_ev[STAGE_RING] = {};
  bool stage_used[STAGE_RING] = {};
  int stage_next = 0;
  // decode steps replay captured graphs, one per launch configuration
  hipStream_t cap_stream = nullptr;
  std::vector<DecodeGraph> graphs;
  bool use_graphs = true;
  // decode attention form: 0 chosen per step, 1 always split-K, 2 one pass where it exists
  int attn_mode = 0;
  // shortest split-K chunk (positions per workgroup)
  int min_chunk = 32;
  // prefill: q/k norm + RoPE + K/V write in the QKV GEMM's epilogue where it applies
  bool fuse_rope = true;
  bool f8_mfma = true;
  int lo_mask = 3;                // bf16 remainder of the norm outputs: 1 attention input, 2 MLP input            // fp8 weights: prefill Q/K/V and gate/up on fp8 matrix instructions
  // measurement hook: per-launch event pairs, labelled by step
  bool timing = false;
  std::vector<TimedLaunch> timed;
  std::vector<hipEvent_t> ev_free;

  void drop_graphs() {
    for (auto& g : graphs) {
      hipGraphExecDestroy(g.exec);
      hipGraphDestroy(g.graph);
    }
    graphs.clear();
  }

  ~fs_model() {
    hipDeviceSynchronize();
    drop_graphs();
    if (cap_stream) hipStreamDestroy(cap_stream);
    for (auto& t : timed) { hipEventDestroy(t.a); hipEventDestroy(t.b); }
    for (auto e : ev_free) hipEventDestroy(e);
    hipFree(wblob); hipFree(nblob); hipFree(sblob); hipFree(wconv); hipFree(kcache); hipFree(vcache);
    hipFree(w8blob); hipFree(s8blob); hipFree(am_pv); hipFree(am_pi);
    hipFree(rope_cos); hipFree(rope_sin);
    hipFree(x); hipFree(xn); hipFree(qkv); hipFree(qr); hipFree(attn); hipFree(hbuf); hipFree(ascale);
    hipFree(d_pos); hipFree(part); hipFree(kpart);
    hipFree(lm_pv); hipFree(lm_pi); hipFree(logits_tmp); hipFree(sample_scr);
    for (int i = 0; i < STAGE_RING; ++i)
      if (stage_ev[i]) hipEventDestroy(stage_ev[i]);
    if (stage) hipHostFree(stage);
    if (gen_host) hipHostFree(gen_host);
    if (tokerr) hipHostFree(tokerr);
    if (pabort) hipHostFree(pabort);
    hipFree(ptrace);
    hipFree(pex);
    for (auto e : gen_ev)
      if (e) hipEventDestroy(e);
    hipFree(gen_tok);
  }
};

namespace {

int skinny_rows(const fs_model* m) {
  return m->wdt == DT_F8 ? SKINNY_MAX_ROWS_F8 : m->wdt == DT_I8 ? SKINNY_MAX_ROWS_I8 : SKINNY_MAX_ROWS;
}

hipEvent_t take_event(fs_model* m) {
  if (!m->ev_free.empty()) {
    hipEvent_t e = m->ev_free.back();
    m->ev_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Enqueues one kernel launch; in timing mode brackets it with events.
#define LAUNCH(m, label, s, expr)                                     \
  do {                                                                \
    hipEvent_t a_ = nullptr;                                          \
    if ((m)->timing && (a_ = take_event(m)) != nullptr)               \
      HIP_TRY(hipEventRecord(a_, s));                                 \
    HIP_TRY(expr);                                                    \
    if (a_ != nullptr) {                                              \
      hipEvent_t b_ = take_event(m);                                  \
      if (b_ != nullptr) {                                            \
        HIP_TRY(hipEventRecord(b_, s));                               \
        (m)->timed.push_back({label, a_, b_});                        \
      }                                                               \
    }                                                                 \
  } while (0)

fs_status ensure_rows(fs_model* m, long long rows, hipStream_t s) {
  if (rows <= m->scratch_rows) return FS_OK;
  HIP_TRY(hipStreamSynchronize(s));
  m->drop_graphs();   // captured graphs point at the old buffers
  hipFree(m->x); hipFree(m->xn); hipFree(m->qkv); hipFree(m->qr); hipFree(m->attn); hipFree(m->hbuf);
  hipFree(m->ascale);
  m->x = nullptr; m->xn = m->qkv = m->qr = m->attn = m->hbuf = nullptr;
  m->ascale = nullptr;
  m->scratch_rows = 0;
  const fs_config& c = m->cfg;
  const size_t R = (size_t)rows;
  // fp32-sized buffers so either activation dtype fits
  if (dalloc(&m->x, R * c.hidden * 4) != hipSuccess || dalloc(&m->xn, R * c.hidden * 4) != hipSuccess ||
      dalloc(&m->qkv, R * m->qkv_w * 4) != hipSuccess || dalloc(&m->qr, R * m->qw * 4) != hipSuccess ||
      dalloc(&m->attn, R * m->qw * 4) != hipSuccess || dalloc(&m->hbuf, R * c.ffn * 4) != hipSuccess ||
      dalloc(&m->ascale, R * 4) != hipSuccess)
    return fail(FS_ERR_OOM, "activation scratch allocation failed");
  m->scratch_rows = rows;
  return FS_OK;
}

// Copies two host int arrays [n] to d_pos / d_slot through the pinned ring:
// the ring slot mirrors the device layout [positions | slots] (max_seqs each),
// so with positions both go in one copy.
fs_status stage_ints(fs_model* m, const int32_t* a, const int32_t* b, int n, hipStream_t s) {
  const int i = m->stage_next;
  const int ms = m->cfg.max_seqs;
  m->stage_next = (i + 1) % STAGE_RING;
  if (m->stage_used[i]) HIP_TRY(hipEventSynchronize(m->stage_ev[i]));
  int32_t* buf = m->stage + (size_t)i * 2 * ms;
  if (a) std::memcpy(buf, a, sizeof(int32_t) * n);
  std::memcpy(buf + ms, b, sizeof(int32_t) * n);
  if (a)
    HIP_TRY(hipMemcpyAsync(m->d_pos, buf, sizeof(int32_t) * (ms + n), hipMemcpyHostToDevice, s));
  else
    HIP_TRY(hipMemcpyAsync(m->d_slot, buf + ms, sizeof(int32_t) * n, hipMemcpyHostToDevice, s));
  HIP_TRY(hipEventRecord(m->stage_ev[i], s));
  m->stage_used[i] = true;
  return FS_OK;
}

fs_status check_slots(const fs_model* m, const int32_t* slots, int B) {
  std::vector<char> seen(m->cfg.max_seqs, 0);
  for (int i = 0; i < B; ++i) {
    const int s = slots[i];
    if (s < 0 || s >= m->cfg.max_seqs)
      return fail(FS_ERR_INVALID_ARG, "slot " + std::to_string(s) + " out of range");
    if (seen[s]) return fail(FS_ERR_INVALID_ARG, "slot " + std::to_string(s) + " repeated in one call");
    seen[s] = 1;
  }
  return FS_OK;
}

int cpl_ok(int K) { return K % 8 == 0 && K <= 4096; }

// A token ID outside [0, vocab) seen by an earlier call's embedding kernel
// (that sequence's rows were made NaN): reported once, then cleared.
fs_status check_token_error(fs_model* m) {
  volatile int32_t* f = m->tokerr;
  if (f == nullptr || f[0] == 0) return FS_OK;
  const int id = f[1], row = f[2];
  f[0] = 0;
  return fail(FS_ERR_INVALID_ARG, "token ID " + std::to_string(id) + " (row " + std::to_string(row) +
                                      " of an earlier call) is outside [0, vocab); that sequence's logits are NaN");
}

// Final RMSNorm of `rows` rows of x at stride ldx, tied head E . h, and
// optionally the greedy IDs.  logits may be null only when `next` is set.
fs_status head(fs_model* m, const float* xrows, int rows, int ldx, float* logits, int32_t* next,
               hipStream_t s) {
  const fs_config& c = m->cfg;
  if (rows <= GEMV_LOGITS_MAX_M) {
    GemvParams p{};
    p.w = m->embed; p.wscale = m->embed_scale; p.N = c.vocab; p.K = c.hidden;
    p.a = xrows; p.lda = ldx; p.M = rows;
    p.gamma = m->final_norm; p.eps = c.rms_eps;
    p.logits = logits; p.ldo = c.vocab;
    p.part_val = m->lm_pv; p.part_idx = m->lm_pi;
    p.aquant = (m->wdt == DT_F8);
    LAUNCH(m, "head", s, gemv(m->wdt, EPI_LOGITS, p, s));
    if (next)
      LAUNCH(m, "argmax", s, argmax_partials(m->lm_pv, m->lm_pi, gemv_logits_blocks(m->wdt, c.vocab, c.hidden),
                                             rows, next, s));
    return FS_OK;
  }
  float* lg = logits != nullptr ? logits : m->logits_tmp;   // logits_tmp allocated by the caller
  if (m->wdt == DT_BF16) {
    LAUNCH(m, "norm", s, rmsnorm(xrows, rows, c.hidden, ldx, m->final_norm, c.rms_eps, m->xn, DT_BF16, c.hidden, s));
    LAUNCH(m, "head", s, gemm_bf16(GEPI_STORE_F32, m->xn, c.hidden, m->embed, c.hidden, lg, c.vocab, rows,
                                   c.vocab, c.hidden, s));
  } else if (m->wdt == DT_F8) {
    // fp8 head: GEMV over groups of up to 4 rows (each quantized in registers)
    for (int r0 = 0; r0 < rows; r0 += 4) {
      GemvParams p{};
      p.w = m->embed; p.wscale = m->embed_scale; p.N = c.vocab; p.K = c.hidden;
      p.a = xrows + (size_t)r0 * ldx; p.lda = ldx; p.M = std::min(4, rows - r0);
      p.gamma = m->final_norm; p.eps = c.rms_eps;
      p.out = lg + (size_t)r0 * c.vocab; p.ldo = c.vocab;
      p.aquant = 1;
      LAUNCH(m, "head", s, gemv(m->wdt, EPI_STORE, p, s));
    }
  } else {
    // fp32 and int8 heads: GEMV over row groups (int8 codes stream once per 4 rows)
    GemvParams p{};
    p.w = m->embed; p.wscale = m->embed_scale; p.N = c.vocab; p.K = c.hidden;
    p.a = xrows; p.lda = ldx; p.M = rows;
    p.gamma = m->final_norm; p.eps = c.rms_eps;
    p.out = lg; p.ldo = c.vocab;
    LAUNCH(m, "head", s, gemv(m->wdt, EPI_STORE, p, s));
  }
  if (next) LAUNCH(m, "argmax", s, argmax_rows_blocks(lg, rows, c.vocab, c.vocab, m->am_pv, m->am_pi, next, s));
  return FS_OK;
}

fs_status ensure_logits_tmp(fs_model* m) {
  if (m->logits_tmp == nullptr &&
      dalloc(&m->logits_tmp, (size_t)m->cfg.max_seqs * m->cfg.vocab * sizeof(float)) != hipSuccess)
    return fail(FS_ERR_OOM, "logits scratch allocation failed");
  return FS_OK;
}

// Number of K splits for a few-row projection with N outputs: the smallest
// that gives >= 192 workgroups, with every wave's share of K a whole number of
// 64-wide chunks; 1 when the few-row kernel does not take the call.
int ksplit_for(const void* A, int lda, const void* W, int rows, int N, int K, const void* A_lo) {
  if (rows > KSPLIT_MAX_ROWS || !gemm_skinny_ok(GEPI_STORE_F32, A, lda, W, K, rows, N, K, A_lo)) return 1;
  const int slabs = N / 32;
  for (int ks = 1; ks <= KSPLIT_MAX; ++ks)
    if (K % (256 * ks) == 0 && slabs * ks >= 192) return ks;
  return 1;
}

// out-projection-shaped GEMM (N = hidden) into the residual stream: x += A . W^T.
// The few-row form splits K over workgroups and leaves its partials pending
// for the next RMSNorm (norm_in) or flush_partials.
hipError_t resid_proj(fs_model* m, const void* A, int lda, const void* W, int rows, int K, const float* cs,
                      hipStream_t s) {
  const fs_config& c = m->cfg;
  if (m->pend_np != 0) return hipErrorInvalidValue;       // partials would be overwritten
  const int ks = ksplit_for(A, lda, W, rows, c.hidden, K, nullptr);
  if (ks == 1) return gemm_bf16(GEPI_RESID_F32, A, lda, W, K, m->x, c.hidden, rows, c.hidden, K, s, nullptr, cs);
  m->pend_np = ks;
  return gemm_skinny(GEPI_PART_F32, A, lda, W, K, m->kpart, c.hidden, rows, c.hidden, K, s, nullptr, cs, ks);
}

// RMSNorm of x into xn (bf16, optional remainder), first adding pending
// partials.  fp8 weights: xn holds the quantized rows, as exact bf16 values of
// code * power-of-two scale (codes = false) or as the e4m3 codes themselves
// with the scales in m->ascale (codes = true), and no remainder.
hipError_t norm_in(fs_model* m, int rows, const float* gamma, void* lo, hipStream_t s, bool codes = false,
                   bool lo8 = false) {
  const fs_config& c = m->cfg;
  float* qs = (m->wdt == DT_F8) ? m->ascale : nullptr;
  if (qs != nullptr) lo = nullptr;
  const int odt = (qs != nullptr && codes) ? DT_F8 : DT_BF16;
  // lo8: the remainder as e4m3 codes (uint8 [rows, hidden] at lo) with its row
  // scales in m->ascale
  int lo_dt = DT_BF16;
  if (lo8 && lo != nullptr && qs == nullptr) {
    qs = m->ascale;
    lo_dt = DT_F8;
  }
  if (m->pend_np == 0)
    return rmsnorm(m->x, rows, c.hidden, c.hidden, gamma, c.rms_eps, m->xn, odt, c.hidden, s, lo, qs, lo_dt);
  const int np = m->pend_np;
  m->pend_np = 0;
  return rmsnorm_add(m->x, m->kpart, np, rows, c.hidden, c.hidden, gamma, c.rms_eps, m->xn, odt, c.hidden, s,
                     lo, qs, lo_dt);
}

// A GEMV over p.M rows; with fp8 weights the quantizing form (the
// RMSNorm-fused inputs) holds at most 4 rows, so larger calls run in groups
// of 4 rows (each streaming the weights once).
hipError_t gemv_rows(fs_model* m, int epi, GemvParams p, hipStream_t s) {
  if (!p.aquant || p.M <= 4) return gemv(m->wdt, epi, p, s);
  const int M = p.M;
  for (int r0 = 0; r0 < M; r0 += 4) {
    GemvParams q = p;
    q.a = p.a + (size_t)r0 * p.lda;
    q.out = p.out + (size_t)r0 * p.ldo;
    q.M = std::min(4, M - r0);
    const hipError_t e = gemv(m->wdt, epi, q, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// One transformer block over `rows` activation rows in the skinny (GEMV) form.
// attention: a callable that consumes m->qkv (fp32) and fills m->attn (fp32).
template <class Attn>
fs_status block_skinny(fs_model* m, const LayerW& L, int rows, Attn&& attention, hipStream_t s) {
  const fs_config& c = m->cfg;
  GemvParams p{};
  p.eps = c.rms_eps;
  // Q/K/V projection with the input RMSNorm fused in
  p.w = L.wqkv; p.wscale = L.sqkv; p.N = m->qkv_w; p.K = c.hidden;
  p.a = m->x; p.lda = c.hidden; p.M = rows; p.gamma = L.attn_norm;
  p.out = (float*)m->qkv; p.ldo = m->qkv_w;
  p.aquant = (m->wdt == DT_F8);
  LAUNCH(m, "qkv", s, gemv_rows(m, EPI_STORE, p, s));
  m->qkv_src = (const float*)m->qkv;
  m->qkv_np = 1;
  fs_status st = attention();
  if (st != FS_OK) return st;
  // output projection + residual
  p.w = L.wo; p.wscale = L.so; p.N = c.hidden; p.K = m->qw;
  p.a = (const float*)m->attn; p.lda = m->qw; p.gamma = nullptr;
  p.out = m->x; p.ldo = c.hidden;
  p.aquant = 0;
  LAUNCH(m, "o_proj", s, gemv(m->wdt, EPI_RESID, p, s));
  // RMSNorm + gate/up + SwiGLU
  p.w = L.wgu; p.wscale = L.sgu; p.N = c.ffn; p.K = c.hidden;
  p.a = m->x; p.lda = c.hidden; p.gamma = L.mlp_norm;
  p.out = (float*)m->hbuf; p.ldo = c.ffn;
  p.aquant = (m->wdt == DT_F8);
  LAUNCH(m, "gate_up", s, gemv_rows(m, EPI_SWIGLU, p, s));
  // down projection + residual
  p.w = L.wdown; p.wscale = L.sdown; p.N = c.hidden; p.K = c.ffn;
  p.a = (const float*)m->hbuf; p.lda = c.ffn; p.gamma = nullptr;
  p.out = m->x; p.ldo = c.hidden;
  p.aquant = 0;
  LAUNCH(m, "down", s, gemv(m->wdt, EPI_RESID, p, s));
  return FS_OK;
}

// One transformer block over `rows` rows in the GEMM (MFMA, bf16) form.  The
// Q/K/V projection is kept in fp32 up to the per-head norm and RoPE (stored
// fp32, or normalised in the large GEMM's epilogue); qkv_f32 marks the decode
// form, whose attention loads the raw fp32 projection itself.
template <class Attn>
fs_status block_gemm(fs_model* m, const LayerW& L, int rows, bool qkv_f32, Attn&& attention,
                     hipStream_t s, const RopeKvParams* rope = nullptr, bool* rope_done = nullptr) {
  const fs_config& c = m->cfg;
  // Both normalised inputs (attention and MLP) keep ~16 significant bits as a
  // bf16 value plus a bf16 remainder (a second MFMA pass over the same weight
  // tiles): with plain bf16 operands at every GEMM input and a 4096-token
  // context the last-token logits reach the whole 2e-2 error budget; the two
  // norm outputs are the largest of those rounding points that the bf16 KV
  // cache does not fix.  On the large GEMM (prefill) the remainder is stored
  // as e4m3 codes with a row scale and multiplied by the fp8 copy of the
  // weights (lo8): twice the K per stage of a bf16 pass, so half its cost, and
  // the remainder (~2^-9 of the value) keeps ~2^-4 relative accuracy.
  void* xn_lo_buf = (m->wdt == DT_F8) ? nullptr : (char*)m->xn + (size_t)rows * c.hidden * 2;
  void* xn_lo = (m->lo_mask & 1) ? xn_lo_buf : nullptr;          // attention input
  void* xn_lo_mlp = (m->lo_mask & 2) ? xn_lo_buf : nullptr;      // MLP input
  // int8 / fp8 weights: each matrix's codes are widened to bf16 (exact) into
  // wconv just before its GEMM, and the row scales are applied per output column
  const bool q8 = (m->wdt == DT_I8 || m->wdt == DT_F8);
  auto widen = [&](const void* codes, size_t n) -> hipError_t {
    return m->wdt == DT_F8 ? f8codes_to_bf16((const uint8_t*)codes, n, m->wconv, s)
                           : codes_to_bf16((const int8_t*)codes, n, m->wconv, s);
  };
  // fp8 weights at prefill sizes: the Q/K/V and gate/up products take the
  // quantized norm outputs as e4m3 codes on the fp8 matrix instructions
  // (gemm_f8); the output and down projections stay weight-only (widened)
  const bool f8mm = m->wdt == DT_F8 && m->f8_mfma && !qkv_f32 && rows >= F8_GEMM_MIN_ROWS &&
                    gemm_f8_ok(GEPI_STORE_F32, m->xn, c.hidden, L.wqkv, c.hidden, m->qkv, m->qkv_w, rows, m->qkv_w,
                               c.hidden) &&
                    gemm_f8_ok(GEPI_SWIGLU_BF16, m->xn, c.hidden, L.wgu, c.hidden, m->hbuf, c.ffn, rows, 2 * c.ffn,
                               c.hidden);
  if (f8mm) {
    LAUNCH(m, "norm", s, norm_in(m, rows, L.attn_norm, nullptr, s, true));
    m->qkv_src = (const float*)m->qkv;
    m->qkv_np = 1;
    if (rope != nullptr && m->fuse_rope && gemm_dma_rope_ok(*rope, rows, m->qkv_w)) {
      LAUNCH(m, "qkv", s, gemm_f8(GEPI_QKV_ROPE, m->xn, c.hidden, L.wqkv, c.hidden, nullptr, 0, rows, m->qkv_w,
                                  c.hidden, s, m->ascale, L.sqkv, rope));
      if (rope_done != nullptr) *rope_done = true;
    } else {
      LAUNCH(m, "qkv", s, gemm_f8(GEPI_STORE_F32, m->xn, c.hidden, L.wqkv, c.hidden, m->qkv, m->qkv_w, rows,
                                  m->qkv_w, c.hidden, s, m->ascale, L.sqkv));
    }
    fs_status st = attention();
    if (st != FS_OK) return st;
    LAUNCH(m, "wconv", s, widen(L.wo, (size_t)c.hidden * m->qw));
    LAUNCH(m, "o_proj", s, resid_proj(m, m->attn, m->qw, m->wconv, rows, m->qw, L.so, s));
    LAUNCH(m, "norm", s, norm_in(m, rows, L.mlp_norm, nullptr, s, true));
    LAUNCH(m, "gate_up", s, gemm_f8(GEPI_SWIGLU_BF16, m->xn, c.hidden, L.wgu, c.hidden, m->hbuf, c.ffn, rows,
                                    2 * c.ffn, c.hidden, s, m->ascale, L.sgu));
    LAUNCH(m, "wconv", s, widen(L.wdown, (size_t)c.hidden * c.ffn));
    LAUNCH(m, "down", s, resid_proj(m, m->hbuf, c.ffn, m->wconv, rows, c.ffn, L.sdown, s));
    return FS_OK;
  }
  const void* wb = L.wqkv;
  if (q8) {
    LAUNCH(m, "wconv", s, widen(L.wqkv, (size_t)m->qkv_w * c.hidden));
    wb = m->wconv;
  }
  const bool lo8_qkv = !q8 && m->lo8 && xn_lo != nullptr && !qkv_f32 &&
                       gemm_dma_ok(GEPI_STORE_F32, m->xn, c.hidden, L.wqkv, c.hidden, m->qkv, m->qkv_w, rows,
                                   m->qkv_w, c.hidden, nullptr);
  LAUNCH(m, "norm", s, norm_in(m, rows, L.attn_norm, xn_lo, s, false, lo8_qkv));
  // decode (fp32 q/k/v): the few-row form splits K in two and the attention
  // sums the partials as it loads q/k/v (not for the gated variant, whose gate
  // rows are read from m->qkv afterwards)
  const int qks = (qkv_f32 && !m->gated)
                      ? std::min(2, ksplit_for(m->xn, c.hidden, wb, rows, m->qkv_w, c.hidden, xn_lo))
                      : 1;
  m->qkv_src = (const float*)m->qkv;
  m->qkv_np = 1;
  if (qks > 1) {
    LAUNCH(m, "qkv", s, gemm_skinny(GEPI_PART_F32, m->xn, c.hidden, wb, c.hidden, m->kpart, m->qkv_w, rows,
                                    m->qkv_w, c.hidden, s, xn_lo, L.sqkv, qks));
    m->qkv_src = m->kpart;
    m->qkv_np = qks;
  } else if (lo8_qkv) {
    const Lo8Params l8{(const uint8_t*)xn_lo, m->ascale, L.w8qkv, L.s8qkv};
    if (rope != nullptr && m->fuse_rope && gemm_dma_rope_ok(*rope, rows, m->qkv_w)) {
      LAUNCH(m, "qkv", s, gemm_dma(GEPI_QKV_ROPE, m->xn, c.hidden, wb, c.hidden, nullptr, 0, rows, m->qkv_w,
                                   c.hidden, s, nullptr, L.sqkv, rope, &l8));
      if (rope_done != nullptr) *rope_done = true;
    } else {
      LAUNCH(m, "qkv", s, gemm_dma(GEPI_STORE_F32, m->xn, c.hidden, wb, c.hidden, m->qkv, m->qkv_w, rows,
                                   m->qkv_w, c.hidden, s, nullptr, L.sqkv, nullptr, &l8));
    }
  } else if (rope != nullptr && m->fuse_rope && !qkv_f32 &&
             gemm_dma_ok(GEPI_QKV_ROPE, m->xn, c.hidden, wb, c.hidden, nullptr, 0, rows, m->qkv_w, c.hidden,
                         xn_lo) &&
             gemm_dma_rope_ok(*rope, rows, m->qkv_w)) {
    // prefill on the large GEMM: the per-head norm, RoPE and K/V write run in
    // its epilogue (rope_done tells the attention step to skip rope_kv)
    LAUNCH(m, "qkv", s, gemm_dma(GEPI_QKV_ROPE, m->xn, c.hidden, wb, c.hidden, nullptr, 0, rows, m->qkv_w,
                                 c.hidden, s, xn_lo, L.sqkv, rope));
    if (rope_done != nullptr) *rope_done = true;
  } else {
    LAUNCH(m, "qkv", s, gemm_bf16(GEPI_STORE_F32, m->xn, c.hidden, wb, c.hidden, m->qkv, m->qkv_w, rows,
                                  m->qkv_w, c.hidden, s, xn_lo, L.sqkv));
  }
  fs_status st = attention();
  if (st != FS_OK) return st;
  wb = L.wo;
  if (q8) {
    LAUNCH(m, "wconv", s, widen(L.wo, (size_t)c.hidden * m->qw));
    wb = m->wconv;
  }
  LAUNCH(m, "o_proj", s, resid_proj(m, m->attn, m->qw, wb, rows, m->qw, L.so, s));
  wb = L.wgu;
  if (q8) {
    LAUNCH(m, "wconv", s, widen(L.wgu, (size_t)2 * c.ffn * c.hidden));
    wb = m->wconv;
  }
  const bool lo8_gu = !q8 && m->lo8 && xn_lo_mlp != nullptr &&
                      gemm_dma_ok(GEPI_SWIGLU_BF16, m->xn, c.hidden, L.wgu, c.hidden, m->hbuf, c.ffn, rows,
                                  2 * c.ffn, c.hidden, nullptr);
  LAUNCH(m, "norm", s, norm_in(m, rows, L.mlp_norm, xn_lo_mlp, s, false, lo8_gu));
  if (lo8_gu) {
    const Lo8Params l8{(const uint8_t*)xn_lo_mlp, m->ascale, L.w8gu, L.s8gu};
    LAUNCH(m, "gate_up", s, gemm_dma(GEPI_SWIGLU_BF16, m->xn, c.hidden, wb, c.hidden, m->hbuf, c.ffn, rows,
                                     2 * c.ffn, c.hidden, s, nullptr, L.sgu, nullptr, &l8));
  } else {
    LAUNCH(m, "gate_up", s, gemm_bf16(GEPI_SWIGLU_BF16, m->xn, c.hidden, wb, c.hidden, m->hbuf, c.ffn, rows,
                                      2 * c.ffn, c.hidden, s, xn_lo_mlp, L.sgu));
  }
  wb = L.wdown;
  if (q8) {
    LAUNCH(m, "wconv", s, widen(L.wdown, (size_t)c.hidden * c.ffn));
    wb = m->wconv;
  }
  LAUNCH(m, "down", s, resid_proj(m, m->hbuf, c.ffn, wb, rows, c.ffn, L.sdown, s));
  return FS_OK;
}

// Adds split-K partials still pending to x (rows rows) without normalising.
fs_status flush_partials(fs_model* m, int rows, hipStream_t s) {
  if (m->pend_np == 0) return FS_OK;
  const fs_config& c = m->cfg;
  const int np = m->pend_np;
  m->pend_np = 0;
  LAUNCH(m, "norm", s, rmsnorm_add(m->x, m->kpart, np, rows, c.hidden, c.hidden, nullptr, c.rms_eps, nullptr,
                                   DT_BF16, c.hidden, s));
  return FS_OK;
}

}  // namespace

// ===================================================================== C ABI
extern "C" {

const char* fs_last_error(void) { return g_err.c_str(); }

fs_status fs_model_create(const fs_config* cfg, const fs_weights* w, void* stream, fs_model** out) {
  g_err.clear();
  if (out == nullptr) return fail(FS_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (cfg == nullptr || w == nullptr) return fail(FS_ERR_INVALID_ARG, "cfg or weights is NULL");
  const fs_config c = *cfg;
  if (c.dtype != FS_F32 && c.dtype != FS_BF16) return fail(FS_ERR_UNSUPPORTED, "unknown dtype");
  if (c.n_layers < 0 || c.hidden <= 0 || c.n_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 ||
      c.ffn <= 0 || c.vocab <= 0 || c.max_seqs <= 0 || c.max_ctx <= 0)
    return fail(FS_ERR_INVALID_ARG, "non-positive size in config");
  if (c.n_heads % c.n_kv_heads != 0) return fail(FS_ERR_INVALID_ARG, "n_heads % n_kv_heads != 0");
  const int rep = c.n_heads / c.n_kv_heads;
  if (rep != 1 && rep != 2 && rep != 4 && rep != 8)
    return fail(FS_ERR_UNSUPPORTED, "n_heads / n_kv_heads must be 1, 2, 4 or 8");
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256)
    return fail(FS_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (c.rope_dim < 0 || c.rope_dim > c.head_dim || c.rope_dim % 16 != 0)
    return fail(FS_ERR_UNSUPPORTED, "rope_dim must be 0 or a multiple of 16 up to head_dim");
  if (c.attn_gate != 0 && c.attn_gate != 1) return fail(FS_ERR_INVALID_ARG, "attn_gate must be 0 or 1");
  if (c.weight_format != FS_WEIGHTS_DTYPE && c.weight_format != FS_WEIGHTS_I8_ROW &&
      c.weight_format != FS_WEIGHTS_F8_ROW)
    return fail(FS_ERR_UNSUPPORTED, "unknown weight_format");
  if (c.hidden % 64 != 0 || c.ffn % 64 != 0)
    return fail(FS_ERR_UNSUPPORTED, "hidden and ffn must be multiples of 64");
  if (!cpl_ok(c.hidden) || !cpl_ok(c.ffn) || !cpl_ok(c.n_heads * c.head_dim))
    return fail(FS_ERR_UNSUPPORTED, "hidden, ffn and n_heads*head_dim must be <= 4096");
  if (!(c.rms_eps >= 0.f) || !(c.rope_theta > 0.f)) return fail(FS_ERR_INVALID_ARG, "bad rms_eps or rope_theta");
  if (w->embed == nullptr || w->final_norm == nullptr || (c.n_layers > 0 && w->layers == nullptr))
    return fail(FS_ERR_INVALID_ARG, "NULL weight pointer");
  const bool q8 = (c.weight_format == FS_WEIGHTS_I8_ROW || c.weight_format == FS_WEIGHTS_F8_ROW);
  const bool f8w = (c.weight_format == FS_WEIGHTS_F8_ROW);
  for (int l = 0; l < c.n_layers; ++l) {
    const fs_layer_weights& L = w->layers[l];
    const void* ps[] = {L.attn_norm, L.wq, L.wk, L.wv, L.q_norm, L.k_norm, L.wo, L.mlp_norm, L.w_gate, L.w_up, L.w_down};
    for (const void* p : ps)
      if (p == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL weight pointer in layer " + std::to_string(l));
    // the quantizer reads matrices in 16-byte vectors
    const void* mats[] = {L.wq, L.wk, L.wv, L.wo, L.w_down};
    for (const void* p : mats)
      if (q8 && ((uintptr_t)p & 15))
        return fail(FS_ERR_INVALID_ARG, "8-bit weights need 16-byte aligned matrices (layer " + std::to_string(l) + ")");
  }
  if (q8 && ((uintptr_t)w->embed & 15)) return fail(FS_ERR_INVALID_ARG, "8-bit weights need a 16-byte aligned embed");
  hipStream_t s = (hipStream_t)stream;
  int device = 0;
  HIP_TRY(hipGetDevice(&device));
  fs_model* m = new fs_model();
  m->cfg = c;
  m->device = device;
  m->dt = c.dtype;
  m->esz = dt_size(c.dtype);
  m->qw = c.n_heads * c.head_dim;
  m->kvw = c.n_kv_heads * c.head_dim;
  m->rot = c.rope_dim > 0 ? c.rope_dim : c.head_dim;
  m->gated = c.attn_gate;
  m->qpw = m->qw * (m->gated ? 2 : 1);          // q (+ gate) projection rows
  m->qkv_w = m->qpw + 2 * m->kvw;
  m->wdt = f8w ? DT_F8 : q8 ? DT_I8 : m->dt;
  const size_t H = c.hidden, I = c.ffn, V = c.vocab, es = m->esz, wes = dt_size(m->wdt);
  const size_t per_layer = ((size_t)m->qkv_w * H + H * m->qw + 2 * I * H + H * I) * wes;
  const size_t wbytes = V * H * wes + per_layer * c.n_layers;
  const size_t nfloats = H + (size_t)c.n_layers * (2 * H + 2 * c.head_dim);
  // int8 row scales: each matrix's run starts on a 64-float (256 B) boundary
  auto rup = [](size_t n) { return (n + 63) / 64 * 64; };
  const size_t sfloats = q8 ? rup(V) + (size_t)c.n_layers * (rup(m->qkv_w) + rup(H) + rup(2 * I) + rup(H)) : 0;
  void* pack_tmp = nullptr;       // packed gate/up of one layer before quantization
  auto bail = [&](fs_status st, const std::string& msg) {
    hipFree(pack_tmp);
    delete m;
    return fail(st, msg);
  };
  if (dalloc(&m->wblob, wbytes) != hipSuccess) return bail(FS_ERR_OOM, "weight allocation failed");
  m->wblob_bytes = wbytes;
  if (dalloc(&m->nblob, nfloats * 4) != hipSuccess) return bail(FS_ERR_OOM, "norm allocation failed");
  if (q8) {
    if (dalloc(&m->sblob, sfloats * 4) != hipSuccess || dalloc(&pack_tmp, 2 * I * H * es) != hipSuccess)
      return bail(FS_ERR_OOM, "int8 scale allocation failed");
    if (m->dt == DT_BF16) {
      const size_t most = std::max(std::max((size_t)m->qkv_w * H, H * m->qw), std::max(2 * I * H, H * I));
      if (dalloc(&m->wconv, most * 2) != hipSuccess) return bail(FS_ERR_OOM, "int8 operand allocation failed");
    }
  }
  char* wp = (char*)m->wblob;
  float* np = m->nblob;
  float* sp = m->sblob;
  hipError_t e = hipSuccess;
  auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
  // a [rows, cols] matrix of cfg.dtype into dst: copied, or quantized with its
  // scales taken from the scale blob
  auto put = [&](const void* src, int rows, int cols, void* dst, float** scale) {
    if (!q8) {
      chk(hipMemcpyAsync(dst, src, (size_t)rows * cols * es, hipMemcpyDeviceToDevice, s));
      return;
    }
    if (*scale == nullptr) *scale = sp;     // the matrix's run of scales starts here
    if (f8w) chk(quantize_rows_f8(src, m->dt, rows, cols, (uint8_t*)dst, sp, s));
    else chk(quantize_rows(src, m->dt, rows, cols, (int8_t*)dst, sp, s));
    sp += rows;
  };
  auto close_run = [&](float* start) {
    if (q8) sp = start + rup((size_t)(sp - start));
  };
  m->embed = wp; wp += V * H * wes;
  put(w->embed, (int)V, (int)H, m->embed, &m->embed_scale);
  close_run(m->embed_scale);
  m->final_norm = np; np += H;
  chk(convert_f32(w->final_norm, m->dt, m->final_norm, H, s));
  m->layers.resize(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l) {
    const fs_layer_weights& src = w->layers[l];
    LayerW& L = m->layers[l];
    L.wqkv = wp; wp += (size_t)m->qkv_w * H * wes;
    put(src.wq, m->qpw, (int)H, L.wqkv, &L.sqkv);
    put(src.wk, m->kvw, (int)H, (char*)L.wqkv + (size_t)m->qpw * H * wes, &L.sqkv);
    put(src.wv, m->kvw, (int)H, (char*)L.wqkv + (size_t)(m->qpw + m->kvw) * H * wes, &L.sqkv);
    close_run(L.sqkv);
    L.wo = wp; wp += H * m->qw * wes;
    put(src.wo, (int)H, m->qw, L.wo, &L.so);
    close_run(L.so);
    L.wgu = wp; wp += 2 * I * H * wes;
    if (q8) {
      chk(pack_gate_up(src.w_gate, src.w_up, m->dt, (int)I, (int)H, pack_tmp, s));
      put(pack_tmp, 2 * (int)I, (int)H, L.wgu, &L.sgu);
      close_run(L.sgu);
    } else {
      chk(pack_gate_up(src.w_gate, src.w_up, m->dt, (int)I, (int)H, L.wgu, s));
    }
    L.wdown = wp; wp += H * I * wes;
    put(src.w_down, (int)H, (int)I, L.wdown, &L.sdown);
    close_run(L.sdown);
    L.attn_norm = np; np += H;
    L.mlp_norm = np; np += H;
    L.q_norm = np; np += c.head_dim;
    L.k_norm = np; np += c.head_dim;
    chk(convert_f32(src.attn_norm, m->dt, L.attn_norm, H, s));
    chk(convert_f32(src.mlp_norm, m->dt, L.mlp_norm, H, s));
    chk(convert_f32(src.q_norm, m->dt, L.q_norm, c.head_dim, s));
    chk(convert_f32(src.k_norm, m->dt, L.k_norm, c.head_dim, s));
  }
  if (e != hipSuccess) return bail(FS_ERR_HIP, std::string("weight repack failed: ") + hipGetErrorString(e));

  // Per layer, a bound on every attention score in base 2.  After the per-head
  // RMSNorm a head row has length <= sqrt(d) (the eps only shortens it), the
  // norm weight g scales each element by at most max|g|, and RoPE rotates
  // pairs (length kept), so |q'| <= sqrt(d) max|g_q| and |k'| <= sqrt(d) max|g_k|;
  // the score q'.k' / sqrt(d) in base 2 is at most log2(e) sqrt(d) max|g_q| max|g_k|.
  // The factor 1.01 covers the bf16 rounding of q' and k' (2^-9 each) and the
  // fp32 sums.  The prefill attention uses it as a fixed softmax shift.
  {
    const char* fx = std::getenv("FS_PREFILL_FIXED_SHIFT");
    const bool fixed = !(fx != nullptr && fx[0] == '0');
    std::vector<float> g(2 * (size_t)c.head_dim);
    for (int l = 0; l < c.n_layers && fixed; ++l) {
      LayerW& L = m->layers[l];
      chk(hipMemcpyAsync(g.data(), L.q_norm, c.head_dim * 4, hipMemcpyDeviceToHost, s));
      chk(hipMemcpyAsync(g.data() + c.head_dim, L.k_norm, c.head_dim * 4, hipMemcpyDeviceToHost, s));
      chk(hipStreamSynchronize(s));
      if (e != hipSuccess) break;
      float gq = 0.f, gk = 0.f;
      for (int i = 0; i < c.head_dim; ++i) {
        gq = std::max(gq, std::fabs(g[i]));
        gk = std::max(gk, std::fabs(g[c.head_dim + i]));
      }
      const double b = 1.4426950408889634 * std::sqrt((double)c.head_dim) * gq * gk * 1.01;
      L.qk_bound = std::isfinite(b) ? (float)b : 0.f;
    }
    if (e != hipSuccess) return bail(FS_ERR_HIP, std::string("norm weight read failed: ") + hipGetErrorString(e));
  }

  // bf16 models: fp8 copies of the Q/K/V and gate/up weights, the operands of
  // the large GEMMs' remainder pass (FS_GEMM_REMAINDER_F8=0 keeps that pass in bf16)
  {
    const char* r8 = std::getenv("FS_GEMM_REMAINDER_F8");
    m->lo8 = m->dt == DT_BF16 && m->wdt == DT_BF16 && H % 64 == 0 && !(r8 != nullptr && r8[0] == '0');
  }
  if (m->lo8) {
    const size_t b8 = ((size_t)m->qkv_w * H + 2 * I * H) * c.n_layers;
    const size_t f8 = (rup(m->qkv_w) + rup(2 * I)) * c.n_layers;
    if (dalloc(&m->w8blob, b8) != hipSuccess || dalloc(&m->s8blob, f8 * 4) != hipSuccess)
      return bail(FS_ERR_OOM, "fp8 weight copy allocation failed");
    uint8_t* bp = (uint8_t*)m->w8blob;
    float* fp = m->s8blob;
    for (int l = 0; l < c.n_layers; ++l) {
      LayerW& L = m->layers[l];
      L.w8qkv = bp; bp += (size_t)m->qkv_w * H;
      L.s8qkv = fp; fp += rup(m->qkv_w);
      L.w8gu = bp; bp += 2 * I * H;
      L.s8gu = fp; fp += rup(2 * I);
      chk(quantize_rows_f8(L.wqkv, DT_BF16, m->qkv_w, (int)H, L.w8qkv, L.s8qkv, s));
      chk(quantize_rows_f8(L.wgu, DT_BF16, 2 * (int)I, (int)H, L.w8gu, L.s8gu, s));
    }
    if (e != hipSuccess) return bail(FS_ERR_HIP, std::string("fp8 weight copy failed: ") + hipGetErrorString(e));
  }

  // KV cache
  m->head_stride = (long long)c.max_ctx * c.head_dim;
  m->slot_stride = m->head_stride * c.n_kv_heads;
  m->layer_stride = m->slot_stride * c.max_seqs;
  const size_t kvbytes = (size_t)m->layer_stride * std::max(c.n_layers, 1) * es;
  if (dalloc(&m->kcache, kvbytes) != hipSuccess || dalloc(&m->vcache, kvbytes) != hipSuccess)
    return bail(FS_ERR_OOM, "KV cache allocation failed");

  // RoPE tables: angle p * theta^(-2i/r) (r = rotated dims) in double, cos/sin stored as fp32
  const int half = m->rot / 2;
  std::vector<float> hc((size_t)c.max_ctx * half), hs((size_t)c.max_ctx * half);
  for (int p = 0; p < c.max_ctx; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * std::pow((double)c.rope_theta, -2.0 * i / (double)m->rot);
      hc[(size_t)p * half + i] = (float)std::cos(ang);
      hs[(size_t)p * half + i] = (float)std::sin(ang);
    }
  if (dalloc(&m->rope_cos, hc.size() * 4) != hipSuccess || dalloc(&m->rope_sin, hs.size() * 4) != hipSuccess)
    return bail(FS_ERR_OOM, "RoPE table allocation failed");
  chk(hipMemcpyAsync(m->rope_cos, hc.data(), hc.size() * 4, hipMemcpyHostToDevice, s));
  chk(hipMemcpyAsync(m->rope_sin, hs.data(), hs.size() * 4, hipMemcpyHostToDevice, s));

  // decode scratch
  m->max_chunks = (c.max_ctx + 31) / 32;
  const int lm_blocks = gemv_logits_blocks(m->wdt, c.vocab, c.hidden);
  if (dalloc(&m->d_pos, (size_t)2 * c.max_seqs * 4) != hipSuccess ||
      dalloc(&m->part, (size_t)c.max_seqs * c.n_heads * m->max_chunks * (c.head_dim + 2) * 4) != hipSuccess ||
      dalloc(&m->kpart, (size_t)KSPLIT_MAX_ROWS * std::max(KSPLIT_MAX * c.hidden, KSPLIT_MAX * m->qkv_w) * 4) !=
          hipSuccess ||
      dalloc(&m->lm_pv, (size_t)GEMV_LOGITS_MAX_M * lm_blocks * 4) != hipSuccess ||
      dalloc(&m->am_pv, (size_t)c.max_seqs * ARGMAX_BLOCKS * 4) != hipSuccess ||
      dalloc(&m->am_pi, (size_t)c.max_seqs * ARGMAX_BLOCKS * 4) != hipSuccess ||
      dalloc(&m->lm_pi, (size_t)GEMV_LOGITS_MAX_M * lm_blocks * 4) != hipSuccess)
    return bail(FS_ERR_OOM, "decode scratch allocation failed");
  m->d_slot = m->d_pos + c.max_seqs;
  if (hipHostMalloc((void**)&m->stage, sizeof(int32_t) * 2 * c.max_seqs * STAGE_RING, hipHostMallocDefault) !=
      hipSuccess)
    return bail(FS_ERR_OOM, "pinned staging allocation failed");
  if (hipHostMalloc((void**)&m->tokerr, 4 * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent) !=
      hipSuccess)
    return bail(FS_ERR_OOM, "pinned token-report allocation failed");
  std::memset(m->tokerr, 0, 4 * sizeof(int32_t));
  chk(hipHostGetDevicePointer((void**)&m->tokerr_dev, m->tokerr, 0));
  for (int i = 0; i < STAGE_RING; ++i) chk(hipEventCreateWithFlags(&m->stage_ev[i], hipEventDisableTiming));
  chk(hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking));
  {
    const char* env = std::getenv("FS_DECODE_GRAPHS");
    if (env != nullptr && env[0] == '0') m->use_graphs = false;
    const char* am = std::getenv("FS_DECODE_ATTN");
    if (am != nullptr && std::strcmp(am, "split") == 0) m->attn_mode = 1;
    if (am != nullptr && std::strcmp(am, "onepass") == 0) m->attn_mode = 2;
    const char* fr = std::getenv("FS_PREFILL_FUSE_ROPE");
    if (fr != nullptr && fr[0] == '0') m->fuse_rope = false;
    const char* lm = std::getenv("FS_GEMM_NORM_REMAINDER");
    if (lm != nullptr && lm[0] >= '0' && lm[0] <= '3' && lm[1] == 0) m->lo_mask = lm[0] - '0';
    const char* f8 = std::getenv("FS_PREFILL_F8_MFMA");
    if (f8 != nullptr && f8[0] == '0') m->f8_mfma = false;
    const char* mc = std::getenv("FS_DECODE_MIN_CHUNK");
    if (mc != nullptr) {
      const int v = std::atoi(mc);
      if (v == 32 || v == 64 || v == 128 || v == 256) m->min_chunk = v;
    }
    // the persistent decode step (opt-in: measured slower than the graph of
    // per-product kernels) needs the 0.6B shape, bf16 weights and all 256 CUs
    // for its 256 resident workgroups
    const char* pe = std::getenv("FS_DECODE_PERSIST");
    int cus = 0;
    chk(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device));
    m->use_persist = (pe != nullptr && pe[0] == '1') && cus == 256 &&
                     decode_persist_ok(c.n_layers, c.hidden, c.n_heads, c.n_kv_heads, c.head_dim, c.ffn, m->dt,
                                       m->wdt, m->gated, m->rot);
    if (m->use_persist) {
      if (dalloc(&m->pex, decode_persist_exchange_bytes()) != hipSuccess)
        return bail(FS_ERR_OOM, "decode exchange allocation failed");
      chk(hipMemsetAsync(m->pex, 0, decode_persist_exchange_bytes(), s));
      if (hipHostMalloc((void**)&m->pabort, 4 * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent) !=
          hipSuccess)
        return bail(FS_ERR_OOM, "pinned abort-word allocation failed");
      std::memset(m->pabort, 0, 4 * sizeof(int32_t));
      chk(hipHostGetDevicePointer((void**)&m->pabort_dev, m->pabort, 0));
      const char* tr = std::getenv("FS_DECODE_TRACE");
      if (tr != nullptr && tr[0] == '1') {
        if (dalloc(&m->ptrace, 1024 * sizeof(long long)) != hipSuccess)
          return bail(FS_ERR_OOM, "trace allocation failed");
        chk(hipMemsetAsync(m->ptrace, 0, 1024 * sizeof(long long), s));
      }
    }
  }
  chk(hipStreamSynchronize(s));
  if (e != hipSuccess) return bail(FS_ERR_HIP, std::string("model setup failed: ") + hipGetErrorString(e));
  hipFree(pack_tmp);
  pack_tmp = nullptr;
  m->slot_len.assign(c.max_seqs, 0);
  *out = m;
  return FS_OK;
}

void fs_model_destroy(fs_model* m) { delete m; }

int32_t fs_slot_length(const fs_model* m, int32_t slot) {
  if (m == nullptr || slot < 0 || slot >= m->cfg.max_seqs) return -1;
  return m->slot_len[slot];
}

fs_status fs_prefill(fs_model* m, const int32_t* tokens, int32_t B, int32_t S, const int32_t* slots,
                     float* logits, void* stream) {
  g_err.clear();
  if (m == nullptr || tokens == nullptr || slots == nullptr || logits == nullptr)
    return fail(FS_ERR_INVALID_ARG, "NULL argument");
  const fs_config& c = m->cfg;
  if (B <= 0 || B > c.max_seqs) return fail(FS_ERR_INVALID_ARG, "B out of range");
  if (S <= 0) return fail(FS_ERR_INVALID_ARG, "empty prompt (S <= 0)");
  if (S > c.max_ctx) return fail(FS_ERR_CAPACITY, "prompt longer than max_ctx");
  fs_status st = check_slots(m, slots, B);
  if (st != FS_OK) return st;
  if ((st = check_token_error(m)) != FS_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const long long T = (long long)B * S;
  if (T > (1LL << 31) / std::max(m->qkv_w, c.ffn)) return fail(FS_ERR_UNSUPPORTED, "B*S too large");
  if ((st = ensure_rows(m, T, s)) != FS_OK) return st;
  if ((st = stage_ints(m, nullptr, slots, B, s)) != FS_OK) return st;
  if (m->timing) LAUNCH(m, "gate", s, spin_wait(TIMING_GATE_US, s));
  LAUNCH(m, "embed", s, embed(m->embed, m->wdt, tokens, (int)T, c.hidden, c.vocab, m->x, s, m->embed_scale,
                              m->tokerr_dev));
  const bool skinny = (m->dt == DT_F32) || T <= skinny_rows(m);
  const int act_dt = skinny ? DT_F32 : DT_BF16;
  m->pend_np = 0;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = m->layers[l];
    char* kc = (char*)m->kcache + (size_t)l * m->layer_stride * m->esz;
    char* vc = (char*)m->vcache + (size_t)l * m->layer_stride * m->esz;
    AttnPrefillParams a{};
    a.q = m->qr; a.q_dt = act_dt; a.kcache = kc; a.vcache = vc; a.kv_dt = m->dt;
    a.out = m->attn; a.o_dt = act_dt; a.slots = m->d_slot;
    a.B = B; a.S = S; a.nq = c.n_heads; a.nkv = c.n_kv_heads; a.d = c.head_dim;
    a.slot_stride = m->slot_stride; a.head_stride = m->head_stride;
    a.scale = 1.0f / std::sqrt((float)c.head_dim);
    // short prompts (up to ATTN_VEC_MAX_S tokens per sequence) keep the vector
    // attention on the GEMM path too: the MFMA kernels' fixed cost dominates
    // there; the head_dim-128 kernel takes q pre-multiplied by scale * log2(e)
    const bool vec = skinny || S <= ATTN_VEC_MAX_S;
    const bool fa = !vec && attn_prefill_fa_ok(a);
    a.q_prescale = fa ? a.scale * 1.4426950408889634f : 1.0f;
    a.m_fixed = L.qk_bound <= ATTN_FIXED_SHIFT_MAX ? L.qk_bound : 0.f;
    RopeKvParams r{};
    r.qscale = a.q_prescale;
    r.rot = m->rot; r.gated = m->gated;
    r.qkv = m->qkv; r.in_dt = DT_F32; r.qout = m->qr; r.q_dt = act_dt;
    r.kcache = kc; r.vcache = vc; r.kv_dt = m->dt;
    r.gq = L.q_norm; r.gk = L.k_norm; r.eps = c.rms_eps;
    r.cos_t = m->rope_cos; r.sin_t = m->rope_sin; r.slots = m->d_slot;
    r.T = (int)T; r.S_per = S; r.nq = c.n_heads; r.nkv = c.n_kv_heads; r.d = c.head_dim;
    r.slot_stride = m->slot_stride; r.head_stride = m->head_stride;
    bool rope_done = false;       // set when the QKV GEMM's epilogue did rope_kv's work
    auto attention = [&]() -> fs_status {
      if (!rope_done) LAUNCH(m, "rope_kv", s, rope_kv(r, s));
      LAUNCH(m, "attn", s, vec ? attn_prefill_vec(a, s) : fa ? attn_prefill_fa(a, s) : attn_prefill(a, s));
      if (m->gated)
        LAUNCH(m, "attn_gate", s, attn_gate(m->attn, act_dt, m->qkv, DT_F32, (int)T, c.n_heads, c.head_dim, m->qkv_w, s));
      return FS_OK;
    };
    st = skinny ? block_skinny(m, L, (int)T, attention, s)
                : block_gemm(m, L, (int)T, false, attention, s, &r, &rope_done);
    if (st != FS_OK) return st;
  }
  if ((st = flush_partials(m, (int)T, s)) != FS_OK) return st;
  // last row of each sequence: rows b*S + S-1
  st = head(m, m->x + (size_t)(S - 1) * c.hidden, B, S * c.hidden, logits, nullptr, s);
  if (st != FS_OK) return st;
  for (int b = 0; b < B; ++b) m->slot_len[slots[b]] = S;
  return FS_OK;
}

// How the decode attention covers the context (longest sequence maxn keys).
// Short contexts at small batch take the one-pass kernel: one 16-wave
// workgroup per (sequence, KV head) and no merge launch (one CU streams the
// head's whole context at ~60 GB/s, so this pays only below ~110 keys).
// Otherwise split-K chunks of at least min_chunk positions, doubled (up to
// 256) while a sequence would need more than 32 chunks (the merge reads up to
// 32 partials in one round trip and loops beyond) or the launch would exceed
// 1024 workgroups; with pow2 the chunk count is rounded up to a power of two
// (chunks past a sequence's end exit at once) so one captured graph serves
// many consecutive positions.
constexpr int ONEPASS_MAX_CTX = 96;
constexpr int SPLIT_MAX_CHUNKS = 32;
constexpr int ONEPASS_MAX_GROUPS = 64;      // B * n_kv_heads
struct AttnSplit {
  int chunk, nchunks;
  bool onepass;
};
static AttnSplit attn_split(const fs_model* m, int B, int maxn, bool pow2, int mode) {
  const fs_config& c = m->cfg;
  const bool can1 = attn_decode_onepass_ok(c.n_heads, c.n_kv_heads, c.head_dim) && !m->gated;
  const bool one = can1 && (mode == 2 || (mode == 0 && maxn <= ONEPASS_MAX_CTX &&
                                          (long long)B * c.n_kv_heads <= ONEPASS_MAX_GROUPS));
  if (one) return {0, 1, true};
  int chunk = m->min_chunk;
  while (chunk < 256 && ((maxn + chunk - 1) / chunk > SPLIT_MAX_CHUNKS ||
                         (long long)((maxn + chunk - 1) / chunk) * c.n_kv_heads * B > 1024))
    chunk *= 2;
  int nchunks = (maxn + chunk - 1) / chunk;
  if (pow2) {
    int p2 = 1;
    while (p2 < nchunks) p2 *= 2;
    nchunks = std::min(p2, (c.max_ctx + chunk - 1) / chunk);
  }
  return {chunk, nchunks, false};
}

// Every kernel of one decode step, in order, on stream s.
static fs_status enqueue_decode(fs_model* m, const int32_t* tokens, int B, float* logits, int32_t* next,
                                const AttnSplit& sp, hipStream_t s) {
  const fs_config& c = m->cfg;
  if (m->timing) LAUNCH(m, "gate", s, spin_wait(TIMING_GATE_US, s));
  LAUNCH(m, "embed", s, embed(m->embed, m->wdt, tokens, B, c.hidden, c.vocab, m->x, s, m->embed_scale,
                              m->tokerr_dev));
  const bool skinny = (m->dt == DT_F32) || B <= skinny_rows(m);
  fs_status st = FS_OK;
  m->pend_np = 0;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = m->layers[l];
    char* kc = (char*)m->kcache + (size_t)l * m->layer_stride * m->esz;
    char* vc = (char*)m->vcache + (size_t)l * m->layer_stride * m->esz;
    auto attention = [&]() -> fs_status {
      AttnDecodeParams a{};
      a.qkv = m->qkv_src; a.qkv_np = m->qkv_np; a.kcache = kc; a.vcache = vc; a.kv_dt = m->dt;
      a.gq = L.q_norm; a.gk = L.k_norm; a.eps = c.rms_eps;
      a.cos_t = m->rope_cos; a.sin_t = m->rope_sin; a.positions = m->d_pos; a.slots = m->d_slot;
      a.part = m->part;
      a.out = sp.onepass ? m->attn : nullptr; a.o_dt = skinny ? DT_F32 : DT_BF16;
      a.B = B; a.nq = c.n_heads; a.nkv = c.n_kv_heads; a.d = c.head_dim; a.chunk = sp.chunk; a.nchunks = sp.nchunks;
      a.slot_stride = m->slot_stride; a.head_stride = m->head_stride;
      a.scale = 1.0f / std::sqrt((float)c.head_dim);
      a.rot = m->rot; a.gated = m->gated;
      LAUNCH(m, "attn", s, attn_decode(a, s));
      // the gated variant's output gate is applied by the merge (the one-pass
      // form is not used for it)
      if (!sp.onepass)
        LAUNCH(m, "combine", s, attn_combine(m->part, m->d_pos, B, c.n_heads, c.head_dim, sp.chunk, sp.nchunks,
                                             m->attn, skinny ? DT_F32 : DT_BF16, s,
                                             m->gated ? (const float*)m->qkv : nullptr, m->qkv_w));
      return FS_OK;
    };
    st = skinny ? block_skinny(m, L, B, attention, s) : block_gemm(m, L, B, true, attention, s);
    if (st != FS_OK) return st;
  }
  if ((st = flush_partials(m, B, s)) != FS_OK) return st;
  return head(m, m->x, B, c.hidden, logits, next, s);
}

fs_status fs_decode_step(fs_model* m, const int32_t* tokens, const int32_t* positions, const int32_t* slots,
                         int32_t B, float* logits, int32_t* next, void* stream) {
  g_err.clear();
  if (m == nullptr || tokens == nullptr || positions == nullptr || slots == nullptr)
    return fail(FS_ERR_INVALID_ARG, "NULL argument");
  if (logits == nullptr && next == nullptr) return fail(FS_ERR_INVALID_ARG, "logits and next are both NULL");
  const fs_config& c = m->cfg;
  if (B <= 0 || B > c.max_seqs) return fail(FS_ERR_INVALID_ARG, "B out of range");
  fs_status st = check_slots(m, slots, B);
  if (st != FS_OK) return st;
  if ((st = check_token_error(m)) != FS_OK) return st;
  int maxn = 0;
  for (int i = 0; i < B; ++i) {
    if (positions[i] != m->slot_len[slots[i]])
      return fail(FS_ERR_INVALID_ARG, "position " + std::to_string(positions[i]) + " != length " +
                                          std::to_string(m->slot_len[slots[i]]) + " of slot " +
                                          std::to_string(slots[i]));
    if (positions[i] >= c.max_ctx) return fail(FS_ERR_CAPACITY, "context exhausted (position >= max_ctx)");
    maxn = std::max(maxn, positions[i] + 1);
  }
  hipStream_t s = (hipStream_t)stream;
  if (m->pabort != nullptr && ((volatile int32_t*)m->pabort)[0] != 0) {
    // a persistent step gave up waiting (workgroups not all resident?): report
    // it once and run later steps on the multi-kernel path
    ((volatile int32_t*)m->pabort)[0] = 0;
    m->use_persist = false;
    return fail(FS_ERR_HIP, "an earlier decode step timed out waiting between workgroups (its logits are "
                            "invalid); later steps use the multi-kernel path");
  }
  if (B == 1 && m->use_persist && maxn <= decode_persist_max_ctx()) {
    const fs_config& cc = m->cfg;
    const LayerW& L0 = m->layers[0];
    DecodePersistParams p{};
    p.wqkv0 = L0.wqkv; p.wo0 = L0.wo; p.wgu0 = L0.wgu; p.wdown0 = L0.wdown;
    p.wstride = cc.n_layers > 1 ? ((const char*)m->layers[1].wqkv - (const char*)L0.wqkv) / 2 : 0;
    p.attn_norm0 = L0.attn_norm; p.mlp_norm0 = L0.mlp_norm; p.q_norm0 = L0.q_norm; p.k_norm0 = L0.k_norm;
    p.nstride = cc.n_layers > 1 ? m->layers[1].attn_norm - L0.attn_norm : 0;
    p.embed = m->embed; p.final_norm = m->final_norm;
    p.V = cc.vocab; p.n_layers = cc.n_layers;
    p.eps = cc.rms_eps; p.qscale = 1.0f / std::sqrt((float)cc.head_dim) * 1.4426950408889634f;
    p.kcache = m->kcache; p.vcache = m->vcache;
    p.layer_stride = m->layer_stride; p.slot_stride = m->slot_stride; p.head_stride = m->head_stride;
    p.cos_t = m->rope_cos; p.sin_t = m->rope_sin;
    p.tokens = tokens; p.pos = positions[0]; p.slot = slots[0]; p.chunk = (positions[0] + 1 + 31) / 32;
    p.logits = logits; p.next = next;
    p.ex = m->pex;
    m->pstep = (m->pstep + 1) & 0xFFFFFFu;
    if (m->pstep == 0) m->pstep = 1;
    p.step_tag = m->pstep << 8;
    p.abort_host = m->pabort_dev;
    p.tokerr = m->tokerr_dev;
    p.trace = m->ptrace;
    LAUNCH(m, "decode_step", s, decode_persist(p, s));
    m->slot_len[slots[0]] = positions[0] + 1;
    return FS_OK;
  }
  if ((st = ensure_rows(m, B, s)) != FS_OK) return st;
  if (B > GEMV_LOGITS_MAX_M && logits == nullptr && (st = ensure_logits_tmp(m)) != FS_OK) return st;
  if ((st = stage_ints(m, positions, slots, B, s)) != FS_OK) return st;
  const AttnSplit sp = attn_split(m, B, maxn, true, m->attn_mode);
  if (sp.nchunks > m->max_chunks) return fail(FS_ERR_HIP, "internal: chunk count exceeds scratch");
  if (!m->use_graphs || m->timing) {
    if ((st = enqueue_decode(m, tokens, B, logits, next, sp, s)) != FS_OK) return st;
  } else {
    // the one-pass form is keyed as chunk 0 and serves every maxn it covers
    const DecodeKey key{B, sp.chunk, sp.nchunks, tokens, logits, next};
    DecodeGraph* g = nullptr;
    for (auto& e : m->graphs)
      if (e.key == key) { g = &e; break; }
    if (g == nullptr) {
      if (m->graphs.size() >= MAX_GRAPHS) {
        HIP_TRY(hipStreamSynchronize(s));
        m->drop_graphs();
      }
      DecodeGraph ng{key, nullptr, nullptr};
      HIP_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeRelaxed));
      st = enqueue_decode(m, tokens, B, logits, next, sp, m->cap_stream);
      const hipError_t ec = hipStreamEndCapture(m->cap_stream, &ng.graph);
      if (st != FS_OK) {
        if (ng.graph) hipGraphDestroy(ng.graph);
        return st;
      }
      if (ec != hipSuccess) return fail(FS_ERR_HIP, std::string("graph capture failed: ") + hipGetErrorString(ec));
      const hipError_t ei = hipGraphInstantiate(&ng.exec, ng.graph, nullptr, nullptr, 0);
      if (ei != hipSuccess) {
        hipGraphDestroy(ng.graph);
        return fail(FS_ERR_HIP, std::string("graph instantiate failed: ") + hipGetErrorString(ei));
      }
      m->graphs.push_back(ng);
      g = &m->graphs.back();
    }
    HIP_TRY(hipGraphLaunch(g->exec, s));
  }
  for (int i = 0; i < B; ++i) m->slot_len[slots[i]] = positions[i] + 1;
  return FS_OK;
}

fs_status fs_kernel_bench(fs_model* m, const char* label, int32_t slot, int32_t position, int32_t reps,
                          double* avg_us, void* stream) {
  g_err.clear();
  if (m == nullptr || label == nullptr || avg_us == nullptr || reps <= 0)
    return fail(FS_ERR_INVALID_ARG, "NULL argument or reps <= 0");
  const fs_config& c = m->cfg;
  // "attn": the form a batch-1 decode step at this position takes; "attn_split"
  // and "attn_onepass" force one; "combine": the merge launch of the split form
  const bool is_attn = std::strcmp(label, "attn") == 0 || std::strcmp(label, "attn_split") == 0 ||
                       std::strcmp(label, "attn_onepass") == 0;
  if ((is_attn || std::strcmp(label, "combine") == 0) && (slot < 0 || slot >= c.max_seqs || position < 0 || position >= c.max_ctx))
    return fail(FS_ERR_INVALID_ARG, "bad slot or position");
  if (c.n_layers == 0 && std::strcmp(label, "head") != 0) return fail(FS_ERR_INVALID_ARG, "model has no layers");
  hipStream_t s = (hipStream_t)stream;
  fs_status st = ensure_rows(m, 1, s);
  if (st != FS_OK) return st;
  int32_t pos_h[1] = {position}, slot_h[1] = {is_attn ? slot : 0};
  if ((st = stage_ints(m, pos_h, slot_h, 1, s)) != FS_OK) return st;
  const int mode = std::strcmp(label, "attn_split") == 0 || std::strcmp(label, "combine") == 0 ? 1
                   : std::strcmp(label, "attn_onepass") == 0                                   ? 2
                                                                                               : m->attn_mode;
  if (mode == 2 && !attn_decode_onepass_ok(c.n_heads, c.n_kv_heads, c.head_dim))
    return fail(FS_ERR_UNSUPPORTED, "no one-pass decode attention for this head shape");
  const AttnSplit sp = attn_split(m, 1, position + 1, false, mode);
  // one launch per layer (the layer's own weights), `reps` passes over the layers
  auto launch_one = [&](int l, hipStream_t ls) -> fs_status {
    const LayerW& L = m->layers[l];
    GemvParams p{};
    p.eps = c.rms_eps; p.M = 1;
    if (std::strcmp(label, "qkv") == 0) {
      p.w = L.wqkv; p.wscale = L.sqkv; p.N = m->qkv_w; p.K = c.hidden; p.a = m->x; p.lda = c.hidden; p.gamma = L.attn_norm;
      p.out = (float*)m->qkv; p.ldo = m->qkv_w;
      p.aquant = (m->wdt == DT_F8);
      HIP_TRY(gemv(m->wdt, EPI_STORE, p, ls));
    } else if (std::strcmp(label, "o_proj") == 0) {
      p.w = L.wo; p.wscale = L.so; p.N = c.hidden; p.K = m->qw; p.a = (const float*)m->attn; p.lda = m->qw;
      p.out = m->x; p.ldo = c.hidden;
      HIP_TRY(gemv(m->wdt, EPI_RESID, p, ls));
    } else if (std::strcmp(label, "gate_up") == 0) {
      p.w = L.wgu; p.wscale = L.sgu; p.N = c.ffn; p.K = c.hidden; p.a = m->x; p.lda = c.hidden; p.gamma = L.mlp_norm;
      p.out = (float*)m->hbuf; p.ldo = c.ffn;
      p.aquant = (m->wdt == DT_F8);
      HIP_TRY(gemv(m->wdt, EPI_SWIGLU, p, ls));
    } else if (std::strcmp(label, "down") == 0) {
      p.w = L.wdown; p.wscale = L.sdown; p.N = c.hidden; p.K = c.ffn; p.a = (const float*)m->hbuf; p.lda = c.ffn;
      p.out = m->x; p.ldo = c.hidden;
      HIP_TRY(gemv(m->wdt, EPI_RESID, p, ls));
    } else if (std::strcmp(label, "head") == 0) {
      p.w = m->embed; p.wscale = m->embed_scale; p.N = c.vocab; p.K = c.hidden; p.a = m->x; p.lda = c.hidden; p.gamma = m->final_norm;
      p.ldo = c.vocab; p.part_val = m->lm_pv; p.part_idx = m->lm_pi;
      p.aquant = (m->wdt == DT_F8);
      HIP_TRY(gemv(m->wdt, EPI_LOGITS, p, ls));
    } else if (is_attn) {
      AttnDecodeParams a{};
      a.qkv = (const float*)m->qkv; a.qkv_np = 1;
      a.kcache = (char*)m->kcache + (size_t)l * m->layer_stride * m->esz;
      a.vcache = (char*)m->vcache + (size_t)l * m->layer_stride * m->esz;
      a.kv_dt = m->dt; a.gq = L.q_norm; a.gk = L.k_norm; a.eps = c.rms_eps;
      a.cos_t = m->rope_cos; a.sin_t = m->rope_sin; a.positions = m->d_pos; a.slots = m->d_slot;
      a.part = m->part; a.B = 1; a.nq = c.n_heads; a.nkv = c.n_kv_heads; a.d = c.head_dim;
      a.out = sp.onepass ? m->attn : nullptr; a.o_dt = DT_F32;
      a.chunk = sp.chunk; a.nchunks = sp.nchunks; a.slot_stride = m->slot_stride; a.head_stride = m->head_stride;
      a.scale = 1.0f / std::sqrt((float)c.head_dim);
      a.rot = m->rot; a.gated = m->gated;
      HIP_TRY(attn_decode(a, ls));
    } else if (std::strcmp(label, "combine") == 0) {
      HIP_TRY(attn_combine(m->part, m->d_pos, 1, c.n_heads, c.head_dim, sp.chunk, sp.nchunks, m->attn, DT_F32, ls));
    } else if (std::strcmp(label, "empty") == 0) {
      HIP_TRY(empty_launch(256, ls));
    } else if (std::strcmp(label, "mfma") == 0) {
      // 256 workgroups x 8 waves: their 2048 sums go to the split-K partial scratch
      const size_t part_floats = (size_t)c.max_seqs * c.n_heads * m->max_chunks * (c.head_dim + 2);
      if (part_floats < 256 * 8) return fail(FS_ERR_UNSUPPORTED, "model scratch too small for the mfma bench");
      HIP_TRY(mfma_peak_launch(m->part, 256, MFMA_PEAK_ITERS, ls));
    } else if (std::strcmp(label, "hbm") == 0) {
      // the whole weight allocation, once per launch; one word per workgroup
      // to the split-K partial scratch
      const size_t part_floats = (size_t)c.max_seqs * c.n_heads * m->max_chunks * (c.head_dim + 2);
      if (part_floats < 2048) return fail(FS_ERR_UNSUPPORTED, "model scratch too small for the hbm bench");
      HIP_TRY(hbm_read_launch(m->wblob, m->wblob_bytes / 16 * 16, reinterpret_cast<unsigned*>(m->part), 2048, ls));
    } else {
      return fail(FS_ERR_INVALID_ARG, std::string("unknown label ") + label);
    }
    return FS_OK;
  };
  const int per_pass = std::strcmp(label, "head") == 0 ? 1 : c.n_layers;
  hipGraph_t g = nullptr;
  hipGraphExec_t ge = nullptr;
  HIP_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeRelaxed));
  for (int l = 0; l < per_pass && st == FS_OK; ++l) st = launch_one(l, m->cap_stream);
  const hipError_t ec = hipStreamEndCapture(m->cap_stream, &g);
  if (st != FS_OK) { if (g) hipGraphDestroy(g); return st; }
  if (ec != hipSuccess) return fail(FS_ERR_HIP, "capture failed");
  if (hipGraphInstantiate(&ge, g, nullptr, nullptr, 0) != hipSuccess) {
    hipGraphDestroy(g);
    return fail(FS_ERR_HIP, "instantiate failed");
  }
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) e = hipGraphLaunch(ge, s);                 // warm
  if (e == hipSuccess) e = hipEventRecord(a, s);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = hipGraphLaunch(ge, s);
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (a) hipEventDestroy(a);
  if (b) hipEventDestroy(b);
  hipGraphExecDestroy(ge);
  hipGraphDestroy(g);
  if (e != hipSuccess) return fail(FS_ERR_HIP, std::string("kernel bench failed: ") + hipGetErrorString(e));
  *avg_us = (double)ms * 1e3 / ((double)reps * per_pass);
  return FS_OK;
}

fs_status fs_decode_trace(fs_model* m, int64_t* out, int32_t n) {
  g_err.clear();
  if (m == nullptr || out == nullptr || n <= 0 || n > 1024) return fail(FS_ERR_INVALID_ARG, "bad argument");
  if (m->ptrace == nullptr) return fail(FS_ERR_UNSUPPORTED, "no trace (set FS_DECODE_TRACE=1 before creating the model)");
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(out, m->ptrace, (size_t)n * sizeof(long long), hipMemcpyDeviceToHost));
  return FS_OK;
}

fs_status fs_timing(fs_model* m, int32_t enable) {
  g_err.clear();
  if (m == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL model");
  HIP_TRY(hipDeviceSynchronize());
  for (auto& t : m->timed) {
    m->ev_free.push_back(t.a);
    m->ev_free.push_back(t.b);
  }
  m->timed.clear();
  m->timing = enable != 0;
  return FS_OK;
}

fs_status fs_timing_read(fs_model* m, const char* label, double* total_ms, int64_t* launches) {
  g_err.clear();
  if (m == nullptr || label == nullptr || total_ms == nullptr || launches == nullptr)
    return fail(FS_ERR_INVALID_ARG, "NULL argument");
  double tot = 0.0;
  int64_t n = 0;
  for (auto& t : m->timed) {
    if (std::strcmp(t.label, label) != 0) continue;
    HIP_TRY(hipEventSynchronize(t.b));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, t.a, t.b));
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return FS_OK;
}

fs_status fs_argmax(const float* logits, int32_t B, int32_t V, int32_t* out, void* stream) {
  g_err.clear();
  if (logits == nullptr || out == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL argument");
  if (B <= 0 || V <= 0) return fail(FS_ERR_INVALID_ARG, "B and V must be positive");
  HIP_TRY(argmax_rows(logits, B, V, V, out, (hipStream_t)stream));
  return FS_OK;
}

fs_status fs_quantize_rows_i8(const void* src, int32_t dtype, int32_t rows, int32_t cols, int8_t* codes,
                              float* scales, void* stream) {
  g_err.clear();
  if (src == nullptr || codes == nullptr || scales == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL argument");
  if (dtype != FS_F32 && dtype != FS_BF16) return fail(FS_ERR_UNSUPPORTED, "unknown dtype");
  if (rows <= 0 || cols <= 0 || cols % 8 != 0) return fail(FS_ERR_INVALID_ARG, "rows, cols must be > 0, cols % 8 == 0");
  if (((uintptr_t)src & 15) || ((uintptr_t)codes & 7) || ((uintptr_t)scales & 3))
    return fail(FS_ERR_INVALID_ARG, "misaligned src (16 B), codes (8 B) or scales (4 B)");
  HIP_TRY(quantize_rows(src, dtype, rows, cols, codes, scales, (hipStream_t)stream));
  return FS_OK;
}

}  // extern "C"

namespace {

// Checks the sampling arguments shared by fs_sample and fs_sample_noalloc and
// fills the kernel parameters (scratch left to the caller).  *greedy is set
// for temperature 0, which needs no scratch.
fs_status sample_setup(const float* logits, int32_t B, int32_t V, const fs_sampling* sp, const float* u,
                       int32_t* out, int32_t max_rows, SampleParams* p, bool* greedy) {
  if (logits == nullptr || sp == nullptr || out == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL argument");
  if (B <= 0 || B > max_rows) return fail(FS_ERR_INVALID_ARG, "B out of range");
  if (V <= 0) return fail(FS_ERR_INVALID_ARG, "V must be positive");
  const float T = sp->temperature;
  if (!(T >= 0.f) || !std::isfinite(T)) return fail(FS_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  if (sp->top_k < 0) return fail(FS_ERR_INVALID_ARG, "top_k must be >= 0");
  if (!(sp->top_p > 0.f && sp->top_p <= 1.f)) return fail(FS_ERR_INVALID_ARG, "top_p must be in (0, 1]");
  *greedy = (T == 0.f);
  if (*greedy) return FS_OK;
  if (u == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL u");
  *p = SampleParams{};
  p->logits = logits; p->ld = V; p->B = B; p->V = V;
  p->G = std::min(SAMPLE_MAX_BLOCKS, std::max(1, (V + 2047) / 2048));
  p->slice = (V + p->G - 1) / p->G;
  p->sc = 1.4426950408889634f / T;
  p->top_k = sp->top_k; p->top_p = sp->top_p;
  p->u = u; p->out = out;
  return FS_OK;
}

}  // namespace

extern "C" {

fs_status fs_quantize_rows_f8(const void* src, int32_t dtype, int32_t rows, int32_t cols, uint8_t* codes,
                              float* scales, void* stream) {
  g_err.clear();
  if (src == nullptr || codes == nullptr || scales == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL argument");
  if (dtype != FS_F32 && dtype != FS_BF16) return fail(FS_ERR_UNSUPPORTED, "unknown dtype");
  if (rows <= 0 || cols <= 0 || cols % 8 != 0) return fail(FS_ERR_INVALID_ARG, "rows, cols must be > 0, cols % 8 == 0");
  if (((uintptr_t)src & 15) || ((uintptr_t)codes & 7) || ((uintptr_t)scales & 3))
    return fail(FS_ERR_INVALID_ARG, "misaligned src (16 B), codes (8 B) or scales (4 B)");
  HIP_TRY(quantize_rows_f8(src, dtype, rows, cols, codes, scales, (hipStream_t)stream));
  return FS_OK;
}

fs_status fs_gemm_f8(const uint8_t* a_codes, const float* a_scales, const uint8_t* w_codes, const float* w_scales,
                     int32_t M, int32_t N, int32_t K, float* out, void* stream) {
  g_err.clear();
  if (a_codes == nullptr || a_scales == nullptr || w_codes == nullptr || w_scales == nullptr || out == nullptr)
    return fail(FS_ERR_INVALID_ARG, "NULL argument");
  if (M <= 0 || N <= 0 || K <= 0 || K % 64 != 0 || N % 8 != 0)
    return fail(FS_ERR_INVALID_ARG, "M, N, K must be > 0, K % 64 == 0, N % 8 == 0");
  if (((uintptr_t)a_codes & 15) || ((uintptr_t)w_codes & 15) || ((uintptr_t)out & 15) || ((uintptr_t)w_scales & 15) ||
      ((uintptr_t)a_scales & 3))
    return fail(FS_ERR_INVALID_ARG, "misaligned codes, out or w_scales (16 B) or a_scales (4 B)");
  HIP_TRY(gemm_f8(GEPI_STORE_F32, a_codes, K, w_codes, K, out, N, M, N, K, (hipStream_t)stream, a_scales, w_scales));
  return FS_OK;
}

fs_status fs_sample(fs_model* m, const float* logits, int32_t B, int32_t V, const fs_sampling* sp,
                    const float* u, int32_t* out, void* stream) {
  g_err.clear();
  if (m == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL argument");
  SampleParams p{};
  bool greedy = false;
  fs_status st = sample_setup(logits, B, V, sp, u, out, m->cfg.max_seqs, &p, &greedy);
  if (st != FS_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (greedy) {
    HIP_TRY(argmax_rows(logits, B, V, V, out, s));
    return FS_OK;
  }
  if (m->sample_scr == nullptr &&
      dalloc(&m->sample_scr, (size_t)m->cfg.max_seqs * sizeof(SampleRowScratch)) != hipSuccess)
    return fail(FS_ERR_OOM, "sampling scratch allocation failed");
  p.scr = m->sample_scr;
  HIP_TRY(sample_rows(p, s));
  return FS_OK;
}

fs_status fs_sample_noalloc(const float* logits, int32_t B, int32_t V, const fs_sampling* sp, const float* u,
                            int32_t* out, void* stream) {
  g_err.clear();
  if (B > SAMPLE_STATIC_MAX_ROWS)
    return fail(FS_ERR_CAPACITY, "B = " + std::to_string(B) + " exceeds the static sampling scratch of " +
                                     std::to_string(SAMPLE_STATIC_MAX_ROWS) + " rows");
  SampleParams p{};
  bool greedy = false;
  fs_status st = sample_setup(logits, B, V, sp, u, out, SAMPLE_STATIC_MAX_ROWS, &p, &greedy);
  if (st != FS_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (greedy) {
    HIP_TRY(argmax_rows(logits, B, V, V, out, s));
    return FS_OK;
  }
  HIP_TRY(sample_static_scratch(&p.scr));
  HIP_TRY(sample_rows(p, s));
  return FS_OK;
}

fs_status fs_generate(fs_model* m, const int32_t* prompt, int32_t S, int32_t slot, const fs_generation* g,
                      int32_t* out_ids, int32_t* n_out, int32_t* stop_reason, void* stream) {
  g_err.clear();
  if (m == nullptr || prompt == nullptr || g == nullptr || n_out == nullptr || stop_reason == nullptr)
    return fail(FS_ERR_INVALID_ARG, "NULL argument");
  *n_out = 0;
  *stop_reason = FS_STOP_NONE;
  const fs_config& c = m->cfg;
  if (g->max_new_tokens < 0) return fail(FS_ERR_INVALID_ARG, "max_new_tokens must be >= 0");
  if (g->n_eos < 0 || (g->n_eos > 0 && g->eos_ids == nullptr)) return fail(FS_ERR_INVALID_ARG, "bad EOS set");
  if (S <= 0) return fail(FS_ERR_INVALID_ARG, "empty prompt (S <= 0)");
  if (S > c.max_ctx) return fail(FS_ERR_CAPACITY, "prompt longer than max_ctx");
  if (slot < 0 || slot >= c.max_seqs) return fail(FS_ERR_INVALID_ARG, "slot out of range");
  const bool sampled = g->sampling != nullptr && g->sampling->temperature != 0.f;
  if (g->max_new_tokens > 0 && out_ids == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL out_ids");
  if (sampled && g->uniforms == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL uniforms");
  {
    const fs_status te = check_token_error(m);
    if (te != FS_OK) return te;
  }
  if (g->max_new_tokens == 0) {                 // zero budget: no forward pass at all
    *stop_reason = FS_STOP_BUDGET;
    return FS_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  fs_status st;
  if ((st = ensure_logits_tmp(m)) != FS_OK) return st;
  if (m->gen_tok == nullptr && dalloc(&m->gen_tok, sizeof(int32_t)) != hipSuccess)
    return fail(FS_ERR_OOM, "token buffer allocation failed");
  if (m->gen_host == nullptr &&
      hipHostMalloc((void**)&m->gen_host, 2 * sizeof(int32_t), hipHostMallocDefault) != hipSuccess)
    return fail(FS_ERR_OOM, "pinned token buffer allocation failed");
  for (auto& e : m->gen_ev)
    if (e == nullptr) HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  float* lg = m->logits_tmp;
  if ((st = fs_prefill(m, prompt, 1, S, &slot, lg, stream)) != FS_OK) return st;
  // Token i's read-back is requested before the decode step that forwards it,
  // so the host checks token i while that step runs on the device (no idle
  // gap per token).  Whether the step may follow is known before the token
  // is read (budget and context); when token i then stops the loop (an EOS ID
  // or no finite logit) the step already issued is discarded: the slot length
  // goes back to S + i and the stream is drained before returning.
  auto done = [&](fs_status r) {
    const hipError_t e = hipStreamSynchronize(s);
    if (r == FS_OK && e != hipSuccess) return fail(FS_ERR_HIP, std::string("HIP error: ") + hipGetErrorString(e));
    return r;
  };
  for (int i = 0;; ++i) {
    // select token i (greedy after a decode step comes fused with the lm_head)
    if (sampled) {
      if ((st = fs_sample(m, lg, 1, c.vocab, g->sampling, g->uniforms + i, m->gen_tok, stream)) != FS_OK)
        return done(st);
    } else if (i == 0) {
      HIP_TRY(argmax_rows(lg, 1, c.vocab, c.vocab, m->gen_tok, s));
    }
    int32_t* host_tok = m->gen_host + (i & 1);
    HIP_TRY(hipMemcpyAsync(host_tok, m->gen_tok, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    HIP_TRY(hipEventRecord(m->gen_ev[i & 1], s));
    const int32_t pos = S + i;
    const bool forward = (i + 1 < g->max_new_tokens) && (pos < c.max_ctx);   // unless token i stops the loop
    if (forward && (st = fs_decode_step(m, m->gen_tok, &pos, &slot, 1, sampled ? lg : nullptr,
                                        sampled ? nullptr : m->gen_tok, stream)) != FS_OK)
      return done(st);
    HIP_TRY(hipEventSynchronize(m->gen_ev[i & 1]));
    const int32_t tok = *host_tok;
    if (tok < 0) {
      if (forward) m->slot_len[slot] = pos;
      done(FS_OK);
      if ((st = check_token_error(m)) != FS_OK) return st;      // a prompt token out of range
      return fail(FS_ERR_UNSUPPORTED, "no finite logit at step " + std::to_string(i));
    }
    bool eos = false;
    for (int e = 0; e < g->n_eos; ++e) eos = eos || g->eos_ids[e] == tok;
    if (eos) {
      if (forward) m->slot_len[slot] = pos;
      if (g->include_stop_id) out_ids[(*n_out)++] = tok;
      *stop_reason = FS_STOP_EOS;
      return done(FS_OK);
    }
    out_ids[(*n_out)++] = tok;
    if (*n_out == g->max_new_tokens) { *stop_reason = FS_STOP_BUDGET; return done(FS_OK); }
    if (pos >= c.max_ctx) { *stop_reason = FS_STOP_CONTEXT; return done(FS_OK); }
  }
}

fs_status fs_kv_read(const fs_model* m, int32_t layer, int32_t slot, int32_t kv_head, int32_t pos0, int32_t n,
                     void* k_out, void* v_out, void* stream) {
  g_err.clear();
  if (m == nullptr || k_out == nullptr || v_out == nullptr) return fail(FS_ERR_INVALID_ARG, "NULL argument");
  const fs_config& c = m->cfg;
  if (layer < 0 || layer >= c.n_layers || slot < 0 || slot >= c.max_seqs || kv_head < 0 ||
      kv_head >= c.n_kv_heads || pos0 < 0 || n <= 0 || pos0 + n > c.max_ctx)
    return fail(FS_ERR_INVALID_ARG, "kv_read range out of bounds");
  const size_t off = ((size_t)layer * m->layer_stride + (size_t)slot * m->slot_stride +
                      (size_t)kv_head * m->head_stride + (size_t)pos0 * c.head_dim) * m->esz;
  const size_t bytes = (size_t)n * c.head_dim * m->esz;
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(hipMemcpyAsync(k_out, (const char*)m->kcache + off, bytes, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(v_out, (const char*)m->vcache + off, bytes, hipMemcpyDeviceToDevice, s));
  return FS_OK;
}

}  // extern "C"
