// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsk {

// DT_I8: signed 8-bit codes with one fp32 scale per row (weights only);
// DT_F8: e4m3 codes with one power-of-two fp32 scale per row
enum Dt { DT_F32 = 0, DT_BF16 = 1, DT_I8 = 2, DT_F8 = 3 };

inline size_t dt_size(int dt) { return dt == DT_BF16 ? 2 : (dt == DT_I8 || dt == DT_F8) ? 1 : 4; }

// ---------------------------------------------------------------- small ops
// x[t, :] = E[tok[t], :] widened to fp32; DT_I8 rows are multiplied by their
// scale (escale[id]).  An id outside [0, V) gives a NaN row and, when bad is
// set, bad[1] = id, bad[2] = t, then bad[0] = 1.
hipError_t embed(const void* E, int dt, const int32_t* tok, int T, int H, int V,
                 float* x, hipStream_t s, const float* escale = nullptr, int32_t* bad = nullptr);
// Per-row symmetric int8: scale[r] = max|src[r,:]| / 127, codes = rint(src / scale)
// (fp32 quotients, ties to even; zero row -> scale 0).  cols % 8 == 0.
hipError_t quantize_rows(const void* src, int dt, int rows, int cols, int8_t* codes, float* scales,
                         hipStream_t s);
// dst[i] = bf16(codes[i]) (exact: |code| <= 127); n % 16 == 0.
hipError_t codes_to_bf16(const int8_t* codes, size_t n, void* dst, hipStream_t s);
// Per-row fp8: scale[r] = the smallest power of two >= fl32(max|src[r,:]| / 448),
// codes = nearest e4m3 of src / scale (ties to even); zero row -> scale 0.  cols % 8 == 0.
hipError_t quantize_rows_f8(const void* src, int dt, int rows, int cols, uint8_t* codes, float* scales,
                            hipStream_t s);
// dst[i] = bf16(value of e4m3 code i) (exact); n % 16 == 0.
hipError_t f8codes_to_bf16(const uint8_t* codes, size_t n, void* dst, hipStream_t s);
// out[t, :] = x[t*ldx, :] / sqrt(mean(x^2) + eps) * g; out of out_dt at row stride ldo.
// lo (bf16 only, optional): the rounding remainder, y - out, also as bf16.
// qs (optional): the fp8 activation rule instead -- qs[t] = the row's
// power-of-two scale and out = its e4m3 codes (out_dt DT_F8) or the exact
// bf16 values code * scale (DT_BF16).
// lo_dt DT_F8 (with lo and qs): out = bf16(y) and the remainder y - out as e4m3
// codes in lo (uint8, row stride ldo) with qs[t] = the remainder row's
// power-of-two scale (the smallest >= max|remainder| / 448).
hipError_t rmsnorm(const float* x, int T, int H, int ldx, const float* g, float eps,
                   void* out, int out_dt, int ldo, hipStream_t s, void* lo = nullptr, float* qs = nullptr,
                   int lo_dt = DT_BF16);
// The same after adding np (<= RMSNORM_MAX_PARTS) split-K partials to the residual rows:
// x[t, :] += parts[0][t, :] + ... + parts[np-1][t, :] (in that order; parts is
// [np][T][H] dense), written back to x, then normalised into out as above.
// out may be null (the additions only).
constexpr int RMSNORM_MAX_PARTS = 16;
hipError_t rmsnorm_add(float* x, const float* parts, int np, int T, int H, int ldx, const float* g, float eps,
                       void* out, int out_dt, int ldo, hipStream_t s, void* lo = nullptr, float* qs = nullptr,
                       int lo_dt = DT_BF16);
// dst[i] = float(src[i])
hipError_t convert_f32(const void* src, int dt, float* dst, size_t n, hipStream_t s);
// A one-wave kernel that waits about `us` microseconds of device wall clock.
hipError_t spin_wait(int us, hipStream_t s);
// `blocks` workgroups of 256 threads that do nothing (the launch floor)
hipError_t empty_launch(int blocks, hipStream_t s);
// `blocks` workgroups of 8 waves, each wave 4 * iters (iters even) 32x32x16 bf16
// matrix instructions on registers; out gets blocks * 8 floats
constexpr int MFMA_PEAK_ITERS = 2048;
// reads `bytes` (a multiple of 16) from p with 16-byte loads; out gets one word per block
hipError_t hbm_read_launch(const void* p, size_t bytes, unsigned* out, int blocks, hipStream_t s);
hipError_t mfma_peak_launch(float* out, int blocks, int iters, hipStream_t s);
// Packs gate/up [I, H] into blocks of 32 gate rows followed by the matching 32 up rows.
hipError_t pack_gate_up(const void* gate, const void* up, int dt, int I, int H, void* dst,
                        hipStream_t s);

// ---------------------------------------------------------------- GEMV (skinny M)
enum GemvEpi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };
static constexpr int GEMV_LOGITS_MAX_M = 4;

struct GemvParams {
  const void* w;       // [N, K] of dt (SWIGLU: packed gate/up, 2*N rows, N = ffn)
  const float* wscale; // DT_I8: per weight row scale (row dot products are multiplied by it)
  int N, K;            // output features, reduction length
  const float* a;      // activations, M rows at stride lda (fp32)
  int lda, M;
  const float* gamma;  // optional RMSNorm weight [K] applied to each activation row
  float eps;
  float* out;          // STORE/SWIGLU: out[m*ldo + n] = y; RESID: out[m*ldo + n] += y
  int ldo;
  // LOGITS epilogue (M <= GEMV_LOGITS_MAX_M)
  float* logits;       // optional, [M, N] at row stride ldo
  int32_t* next;       // optional [M]: greedy IDs
  float* part_val;     // [M * gemv_logits_blocks] per-block best values
  int32_t* part_idx;   // [M * gemv_logits_blocks] per-block best indices
  int groups;          // set by the launcher
  int aquant;          // DT_F8 with gamma, M <= 4: quantize each normalised activation row to fp8
};
hipError_t gemv(int dt, int epi, GemvParams p, hipStream_t s);
// The DT_F8 part of gemv (its own translation unit).
hipError_t gemv_f8(int epi, GemvParams p, hipStream_t s);
// Number of workgroups (and per-row partials) the LOGITS epilogue uses.
int gemv_logits_blocks(int dt, int N, int K);
// next[m] = best of the nblocks (value, index) partials of row m.
hipError_t argmax_partials(const float* pv, const int32_t* pi, int nblocks, int M, int32_t* next,
                           hipStream_t s);

// ---------------------------------------------------------------- MFMA GEMM (bf16)
enum GemmEpi { GEPI_STORE_BF16 = 0, GEPI_RESID_F32 = 1, GEPI_SWIGLU_BF16 = 2, GEPI_STORE_F32 = 3,
               GEPI_PART_F32 = 4, GEPI_QKV_ROPE = 5 };
// C[M, N] = A[M, K] . B[N, K]^T; A, B bf16 row-major with K contiguous (lda, ldb);
// fp32 accumulation.  STORE_*: out[m*ldc + n] = C; RESID_F32: out[m*ldc + n] += C;
// SWIGLU_BF16: B is packed gate/up (blocks of 32+32 rows, N = 2*ffn) and
// out[m*ldc + f] = silu(gate_f) * up_f.  Requires K % 64 == 0 (and N % 64 == 0 for SWIGLU).
// A_lo (optional): a second bf16 operand of A's shape; C = (A + A_lo) . B^T, the
// remainder pass reusing each B tile (keeps activations near fp32 precision).
// colscale (optional, fp32 [N]): C[:, n] *= colscale[n] before the epilogue
// (B holding int8 codes as bf16, colscale their row scales).
hipError_t gemm_bf16(int epi, const void* A, int lda, const void* B, int ldb, void* out, int ldc,
                     int M, int N, int K, hipStream_t s, const void* A_lo = nullptr,
                     const float* colscale = nullptr);
// The large-problem kernel behind gemm_bf16 (256x256 tiles, operands streamed
// into LDS by DMA): gemm_dma_ok says whether it applies to a call.
// QKV_ROPE (only here): C is a prefill's fused q|k|v projection and never
// stored as such; the epilogue applies rope_kv's per-head q/k RMSNorm + RoPE
// (head_dim 128, full rotation, no output gate, fp32 input, bf16 q and KV) to
// the fp32 products and writes q' and the K/V cache rows as rope_kv would from
// the stored fp32 projection (same bits); gemm_dma_rope_ok says whether a
// rope_kv call qualifies (M = its T, N = its packed width).
bool gemm_dma_ok(int epi, const void* A, int lda, const void* B, int ldb, const void* out, int ldc,
                 int M, int N, int K, const void* A_lo);
struct RopeKvParams;
bool gemm_dma_rope_ok(const RopeKvParams& r, int M, int N);
// The remainder pass of gemm_dma on fp8 operands (instead of A_lo): a [M, K]
// e4m3 codes of the activation remainder with power-of-two row scales as[M],
// b [N, K] an fp8 copy of the weights with row scales bs[N]; the kernel adds
// diag(as) . (a . b^T) . diag(bs) into the same fp32 tile.  K % 64 == 0,
// 16-B aligned code rows.
struct Lo8Params {
  const uint8_t* a; const float* as;
  const uint8_t* b; const float* bs;
};
hipError_t gemm_dma(int epi, const void* A, int lda, const void* B, int ldb, void* out, int ldc,
                    int M, int N, int K, hipStream_t s, const void* A_lo, const float* colscale,
                    const RopeKvParams* rope = nullptr,
                    const Lo8Params* lo8 = nullptr);
// fp8 (e4m3) form of gemm_dma for the fp8 weight option: A [M, K] and B
// [N, K] are e4m3 codes, K contiguous (lda, ldb in bytes, multiples of 16; K a
// multiple of 64), C = diag(rowscale) . (A . B^T) . diag(colscale) in fp32
// (either scale may be null), then the store form epi as for gemm_dma
// (STORE_F32, SWIGLU_BF16 or QKV_ROPE: the quantized-input products).  Any
// M, N >= 1 (tiles past the edges compute on clamped rows and store nothing);
// the caller decides when the 256x256 tiling pays.
bool gemm_f8_ok(int epi, const void* A, int lda, const void* B, int ldb, const void* out, int ldc, int M, int N,
                int K);
hipError_t gemm_f8(int epi, const void* A, int lda, const void* B, int ldb, void* out, int ldc, int M, int N,
                   int K, hipStream_t s, const float* rowscale, const float* colscale,
                   const RopeKvParams* rope = nullptr);

// The few-rows kernel behind gemm_bf16 (M <= 64, K % 256 == 0, N % 32 == 0):
// one weight slab per workgroup, K split over its waves, each weight read once.
// PART_F32 (only here): K is also split over ksplit workgroups per slab
// (K % (256 * ksplit) == 0) and split s stores its partial product at
// out + s * M * ldc (fp32, [ksplit][M][ldc]); rmsnorm_add sums them.
bool gemm_skinny_ok(int epi, const void* A, int lda, const void* B, int ldb, int M, int N, int K,
                    const void* A_lo);
hipError_t gemm_skinny(int epi, const void* A, int lda, const void* B, int ldb, void* out, int ldc, int M, int N,
                       int K, hipStream_t s, const void* A_lo, const float* colscale, int ksplit = 1);

// ---------------------------------------------------------------- q/k norm + RoPE + KV write
// For T tokens: token t belongs to sequence t / S_per (slot slots[t / S_per]) at
// position pos0 + t % S_per (prefill: pos0 = 0).  Reads qkv rows [T, (nq+2nkv)*d]
// of in_dt; writes q' [T, nq*d] of q_dt (RMSNorm over d with g_q, RoPE), and
// K' (RMSNorm with g_k, RoPE), V into the cache of kv_dt.
struct RopeKvParams {
  const void* qkv; int in_dt;
  void* qout; int q_dt;
  void* kcache; void* vcache; int kv_dt;
  const float* gq; const float* gk; float eps;
  const float* cos_t; const float* sin_t;   // [max_ctx, d/2]
  const int32_t* slots;                     // device [B]
  int T, S_per, nq, nkv, d;
  long long slot_stride;                    // elements per (layer, slot)
  long long head_stride;                    // elements per KV head (= max_ctx * d)
  float qscale;                             // factor applied to q' before it is stored (1: none)
  int rot;                                  // rotated dims per head (pairs (i, i + rot/2))
  int gated;                                // q rows interleaved with gate rows per head
};
hipError_t rope_kv(const RopeKvParams& p, hipStream_t s);

// Gated attention output: a[t, h*d + e] *= sigmoid(qkv[t, 2h*d + d + e]) for
// T rows (a of a_dt, [T, nq*d]; qkv of qkv_dt, rows of width ldq).
hipError_t attn_gate(void* a, int a_dt, const void* qkv, int qkv_dt, int T, int nq, int d, int ldq,
                     hipStream_t s);

// ---------------------------------------------------------------- attention
// Prefill: causal attention of T = B*S queries against their slot's cache
// positions 0..p.  q [T, nq*d] of q_dt; out [T, nq*d] of o_dt.
struct AttnPrefillParams {
  const void* q; int q_dt;
  const void* kcache; const void* vcache; int kv_dt;
  void* out; int o_dt;
  const int32_t* slots;        // device [B]
  int B, S, nq, nkv, d;
  long long slot_stride, head_stride;
  float scale;
  float q_prescale;            // factor already applied to q (attn_prefill_fa expects scale*log2(e))
  // attn_prefill_fa: > 0 bounds every base-2 score |q'.k'| * scale * log2(e) of
  // the layer (per-head q/k RMSNorm makes |q'| <= sqrt(d) max|g_q|, likewise k');
  // up to ATTN_FIXED_SHIFT_MAX the softmax needs no running max.  0: running max.
  float m_fixed;
};
// Largest score bound taken without a running max: with |s| <= 63 every
// p = 2^s lies in [2^-63, 2^63], a normal fp32 / bf16 number, unshifted.
constexpr float ATTN_FIXED_SHIFT_MAX = 63.f;
hipError_t attn_prefill(const AttnPrefillParams& p, hipStream_t s);      // MFMA path when bf16
hipError_t attn_prefill_vec(const AttnPrefillParams& p, hipStream_t s);  // vector path, any dtype
// head_dim 128, bf16, even query heads per KV head: 64 queries per wave, K/V
// tiles streamed into LDS by DMA (the kernel behind attn_prefill for that case)
// With that kernel q is stored pre-multiplied by scale*log2(e) (RopeKvParams.qscale,
// AttnPrefillParams.q_prescale); the other attention kernels take q unscaled.
bool attn_prefill_fa_ok(const AttnPrefillParams& p);
hipError_t attn_prefill_fa(const AttnPrefillParams& p, hipStream_t s);

// Decode: one new token per sequence, split over context chunks, with the
// q/k RMSNorm + RoPE + KV append of the new token fused in.  Each workgroup
// writes its chunk's partial (unnormalised o[d], running max m, sum l) for
// the query heads of its KV head; attn_combine merges them.
struct AttnDecodeParams {
  const float* qkv;            // [qkv_np][B, (nq+2nkv)*d] fp32 (raw projections; qkv_np
  int qkv_np;                  //   (1 or 2) split-K partials, summed on load; 1 = the plain rows)
  void* kcache; void* vcache; int kv_dt;
  const float* gq; const float* gk; float eps;
  const float* cos_t; const float* sin_t;
  const int32_t* positions;    // device [B]
  const int32_t* slots;        // device [B]
  float* part;                 // [B, nq, nchunks, d + 2]: o[0..d), m, l (base-2 softmax)
  void* out;                   // non-null: one pass over the whole context, out[b, h*d + e] in o_dt
  int o_dt;                    //   (part, chunk and nchunks unused)
  int B, nq, nkv, d, chunk, nchunks;
  long long slot_stride, head_stride;
  float scale;
  int rot;                     // rotated dims per head
  int gated;                   // q rows interleaved with gate rows per head
};
hipError_t attn_decode(const AttnDecodeParams& p, hipStream_t s);
// The one-pass form exists for (nq/nkv) * d <= ATTN_ONEPASS_MAX_REP_D (its
// 16-wave workgroup keeps q and the output state of every query head of the
// group in registers).
constexpr int ATTN_ONEPASS_MAX_REP_D = 256;
bool attn_decode_onepass_ok(int nq, int nkv, int d);
// out[b, h*d + e] from the chunk partials of sequence b (chunks 0..positions[b]/chunk).
// gate (optional, fp32 rows of width ldg, the gated variant's q projection with
// per-head interleaved [q | gate]): out[b, h*d + e] *= sigmoid(gate[b*ldg + (2h+1)*d + e]).
hipError_t attn_combine(const float* part, const int32_t* positions, int B, int nq, int d, int chunk,
                        int nchunks, void* out, int o_dt, hipStream_t s, const float* gate = nullptr,
                        int ldg = 0);

// ---------------------------------------------------------------- persistent batch-1 decode step
// One launch of 256 workgroups (one per CU, all resident) runs a whole decode
// step of one sequence: embedding, every layer, final norm, tied head, logits
// and/or the greedy ID.  The 0.6B shape only (decode_persist_ok); contexts up
// to decode_persist_max_ctx() keys.  Workgroups hand activations to each other
// through `ex` (decode_persist_exchange_bytes(), zeroed once at allocation),
// records tagged with step_tag (distinct per step, nonzero, low 8 bits 0).  A
// wait that exceeds its bound sets *abort_host (host-mapped) and the ex abort
// word; after that the exchange buffer must be cleared before another launch.
struct DecodePersistParams {
  const void *wqkv0, *wo0, *wgu0, *wdown0;   // layer 0's matrices (bf16, packed as the model stores them)
  long long wstride;                          // elements from one layer's matrices to the next
  const float *attn_norm0, *mlp_norm0, *q_norm0, *k_norm0;
  long long nstride;                          // floats from one layer's norm vectors to the next
  const void* embed;                          // [V, H] bf16, also the head
  const float* final_norm;
  int V, n_layers;
  float eps, qscale;                          // rms eps; 1/sqrt(head_dim) * log2(e)
  void *kcache, *vcache;                      // bf16 [layer][slot][kv head][pos][d]
  long long layer_stride, slot_stride, head_stride;
  const float *cos_t, *sin_t;                 // [max_ctx][d/2]
  const int32_t* tokens;                      // device [1]
  int pos, slot, chunk;                       // chunk = keys per workgroup = ceil((pos + 1) / 32)
  float* logits;                              // device [V] or null
  int32_t* next;                              // device [1] or null
  void* ex;
  unsigned step_tag;
  int32_t* abort_host;                        // host-mapped word
  int32_t* tokerr;                            // host-mapped {flag, id, row} or null
  long long* trace;                           // device [1024] clock stamps of workgroup 0, or null
};
bool decode_persist_ok(int n_layers, int hidden, int n_heads, int n_kv_heads, int head_dim, int ffn, int dt,
                       int wdt, int gated, int rot);
int decode_persist_max_ctx();
size_t decode_persist_exchange_bytes();
hipError_t decode_persist(const DecodePersistParams& p, hipStream_t s);

// ---------------------------------------------------------------- argmax
// out[b] = greedy ID of row b of logits [B, V] (row stride ldl).
hipError_t argmax_rows(const float* logits, int B, int V, int ldl, int32_t* out, hipStream_t s);
// argmax_rows in two levels for many rows: ARGMAX_BLOCKS blocks per row write
// (value, index) bests to pv / pi ([B][ARGMAX_BLOCKS]), then argmax_partials.
constexpr int ARGMAX_BLOCKS = 16;
hipError_t argmax_rows_blocks(const float* logits, int B, int V, int ldl, float* pv, int32_t* pi, int32_t* out,
                              hipStream_t s);

// ---------------------------------------------------------------- sampling
// Per-row scratch of the sampler (count and mass histograms of the three radix
// levels, max key, finite count, per-block kept mass).
constexpr int SAMPLE_MAX_BLOCKS = 128;
struct SampleRowScratch {
  uint32_t c1[4096], c2[4096], c3[256];
  float m1[4096], m2[4096], m3[256];
  uint32_t maxkey, nfinite;
  float bsum[SAMPLE_MAX_BLOCKS];
  // selections made so far (written by block 0 of the pass that makes them)
  uint32_t kb1, kr1, kb2, kr2, kcut;   // top-k digits, remaining counts, the full cut key
  uint32_t pb1, pb2, cut;              // top-p digits and the final cut key
  float z, pr1, pr2;                   // top-k mass, remaining masses
};
struct SampleParams {
  const float* logits; long long ld;   // rows of logits, ld elements apart
  int B, V, G, slice;                  // G blocks of `slice` token IDs per row
  float sc;                            // log2(e) / temperature (temperature > 0)
  int top_k; float top_p;              // 0 = no top-k limit; top_p in (0, 1]
  const float* u;                      // device [B], uniform in [0, 1)
  int32_t* out;                        // device [B]
  SampleRowScratch* scr;               // device [B]
};
// temperature -> top-k -> top-p -> renormalise -> draw for B rows; -1 for a row
// without a finite logit.  Clears p.scr rows 0..B-1 itself (a fill kernel).
hipError_t sample_rows(const SampleParams& p, hipStream_t s);
// Device address, on the current device, of the library's static row scratch
// (SAMPLE_STATIC_MAX_ROWS rows, one copy per device, never freed); looked up
// with hipGetSymbolAddress on the first call per device.  Allocates nothing.
constexpr int SAMPLE_STATIC_MAX_ROWS = 64;
hipError_t sample_static_scratch(SampleRowScratch** out);

}  // namespace fsk
