/* libcsa -- hybrid compressed attention (CSA + HCA) on AMD Instinct MI355X (gfx950).
 *
 * The layer, as described on the pages this library follows:
 *   [csdn]   deepseek.csdn.net "一文搞懂 DeepSeek：从 V3 的 KV 压缩与 MoE，到 V4 的百万 token 上下文",
 *            sections "V3 看家本领一：MLA" (latent KV + decoupled RoPE key, absorbed projections)
 *            and "V4 改进一：CSA 与 HCA" (compress, index, select, attend with window; HCA).
 *   [yudong] yudonglee.me "DeepSeek-V4 详解", 2.2 (CSA Steps 1-4) and 2.3 (HCA Steps 1-2).
 *   [hongke] hongke120.com/20112.html, 2.2-2.3 and 4.1 (four cache entry types: raw tail tokens,
 *            CSA blocks, HCA summaries, indexer keys).
 *   [jaylab] jaylab-temp.pages.dev "DeepSeek-V4 — 百万 Token 上下文的高效 MoE 模型",
 *            其他技术细节 (cache rows: RoPE dims bf16, the rest fp8).
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never allocates and
 *     keeps no state besides its loaded kernels (and the optional, lock-guarded kernel timing
 *     below). Calls that need scratch take (ws, ws_bytes),
 *     sized by the matching *_workspace_bytes() query; ws may be NULL when that query returns 0.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns. No call synchronises. Calls are safe from any host thread.
 *   - Arguments are validated on the host before anything is enqueued; on any error nothing is
 *     enqueued and the outputs are untouched. Device-array contents (positions, sequence ids,
 *     indices) are trusted preconditions.
 *   - Layouts are row-major and dense unless a leading dimension (ld, in elements) says
 *     otherwise. bf16 data is passed as raw 16-bit codes; E4M3 as raw bytes (OCP E4M3FN, max 448).
 *   - The library prints nothing and throws nothing across this boundary.
 *
 * Numerics (per call below): fp32 accumulation everywhere. The MFMA attention paths compute in
 * fp16 on operands converted exactly from bf16 / (fp8 x row scale): they require every cache and
 * query value to have magnitude below 65504 (values under 2^-17 keep at most 2^-25 absolute
 * error). The pages state that queries and KV entries are RMS-normalised before attention
 * (jaylab, Muon bullet list), which keeps them far inside that range.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 2

typedef enum {
  CSA_OK = 0,
  CSA_EINVAL = 1,        /* null pointer, non-positive size, inconsistent arguments          */
  CSA_EUNSUPPORTED = 2,  /* valid request with no kernel (dtype / shape combination)          */
  CSA_EWORKSPACE = 3,    /* ws_bytes smaller than the matching *_workspace_bytes() query      */
  CSA_EHIP = 4           /* a HIP launch failed; csa_last_error() holds the HIP error text    */
} csa_status;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_E4M3 = 2 } csa_dtype;

/* A store of cache rows for B sequences: row = c[d_c] followed by r[d_r] ([csdn] MLA section:
 * the latent and the decoupled RoPE key are cached per token).
 *   c      [B][rows][ld_c] in dtype_c; the first d_c elements of a row are used.
 *   r      [B][rows][ld_r]; bf16 when dtype_c is CSA_BF16 or CSA_E4M3, fp32 when CSA_F32.
 *          May alias c (e.g. r = c + d_c with ld_r = ld_c for an interleaved bf16 row).
 *          NULL iff d_r == 0.
 *   scale  [B][rows] fp32 dequantisation scale of c; required iff dtype_c == CSA_E4M3, else NULL.
 *          The dequantised row is (scale * c, r) ([jaylab] mixed-precision cache row).
 *   pos0   [B] int64 ring offset of a raw-token store; NULL means 0. A raw store is a ring:
 *          position p of sequence b lives in row (p - pos0[b]) mod rows, so a store that holds
 *          every position from pos0 on (rows >= positions held) reads row p - pos0, and a window
 *          store of rows >= window rows is rolled by writing each new token over the oldest row
 *          (csa_cache_append does), with no copy of the others. */
typedef struct {
  const void* c;
  const void* r;
  const float* scale;
  const int64_t* pos0;
  int32_t dtype_c;
  int32_t d_c, d_r;
  int64_t rows;
  int64_t ld_c, ld_r;
} csa_kv_t;

/* The writable twin of csa_kv_t (output of csa_compress; pos0 unused). */
typedef struct {
  void* c;
  void* r;
  float* scale;
  int32_t dtype_c;
  int32_t d_c, d_r;
  int64_t rows;
  int64_t ld_c, ld_r;
} csa_kv_out_t;

/* Queries: nq of them; query i belongs to sequence seq[i] (int32, device) and sits at absolute
 * position pos[i] (int64, device). The pages' causal reading used throughout: entry j of an
 * m-fold compressed store covers positions [j*m, (j+1)*m - 1] and is visible to a query at pos
 * iff (j+1)*m - 1 <= pos, i.e. n_vis(pos) = min(N, floor((pos + 1) / m)). */
typedef struct {
  const int32_t* seq;
  const int64_t* pos;
  int32_t nq;
} csa_queries_t;

/* ---------------------------------------------------------------------------------------------
 * csa_compress -- softmax-gated pooling of every m consecutive token rows into one entry.
 * [csdn] V4 改进一 (CSA step one) and [yudong] 2.2 Step 1 (m = 4); [yudong] 2.3 Step 1 and
 * [hongke] 2.3 (m' = 128, HCA uses the same pooling).
 *   For each sequence b, block j < T/m (a trailing partial block is not emitted) and channel c of
 *   the d = d_c + d_r channels:  a_i = g[b][jm+i][c] + bias[i],  w = softmax_i(a),
 *   e[b][j][c] = sum_i w_i x[b][jm+i][c].
 *   x, g   [B][T][d] in in_dtype (CSA_F32 or CSA_BF16); or NULL in projection mode.
 *   bias   [m] fp32 position bias.
 *   Projection mode (fp32 only): x and g NULL, hidden [B][T][d_model] fp32 and w_x, w_g
 *          [d_model][d] fp32 given; x = hidden * w_x and g = hidden * w_g are formed on the fly
 *          ([csdn] MLA: the cached latent is a projection of the token's input), and x is also
 *          written to raw_x_out [B][T][d] fp32 (the raw rows a sliding window reads).
 *          Otherwise hidden, w_x, w_g and raw_x_out must be NULL.
 *   out    entry store with out->rows == T/m: out->dtype_c CSA_F32, CSA_BF16 (RNE) or CSA_E4M3
 *          (one fp32 scale per row, scale = amax(|e_c|)/448, codes RNE-satfinite of e_c/scale;
 *          an all-zero row stores scale 0). The r part is stored bf16 (fp32 when out is F32).
 *   Constraints: m >= 1, T >= 0, d % 4 == 0 (fp32) or d % 8 == 0 (bf16). Projection mode also
 *   needs d % 64 == 0, an even d_c, d_model % 4 == 0, m in {1, 2, 4}, a non-E4M3 out and 16-byte
 *   aligned hidden, w_x, w_g (CSA_EUNSUPPORTED otherwise).
 * ------------------------------------------------------------------------------------------- */
csa_status csa_compress(const void* x, const void* g, int32_t in_dtype, const float* bias,
                        int32_t m, int32_t B, int64_t T, int32_t d_c, int32_t d_r,
                        const float* hidden, const float* w_x, const float* w_g, int32_t d_model,
                        const csa_kv_out_t* out, float* raw_x_out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * csa_cache_append -- decode-time cache maintenance: one new token per sequence.
 * [csdn] V4 改进一 (CSA step one, HCA) and [yudong] 2.2 Step 1 / 2.3 Step 1 (m consecutive tokens
 * pooled into one entry with position-biased softmax weights); [jaylab] 其他技术细节 (cache rows:
 * fp8 latent with a row scale, bf16 RoPE dims). For every sequence b, with its new token at the
 * absolute position p = pos[b] (int64, device, p >= 0):
 *   - stage_x[b][p % m] = x_new[b] and stage_g[b][p % m] = g_new[b], widened to fp32;
 *   - raw ring row (p - raw_pos0[b]) mod raw->rows (raw_pos0 NULL: 0) of `raw` = x_new[b], stored
 *     like a csa_compress output row (f32 / bf16 / e4m3 latent with sigma = max|latent| / 448;
 *     RoPE bf16, or f32 in an f32 store). raw may be NULL (or have 0 rows): no raw row is stored.
 *     With raw->rows >= the attention window this keeps the window of csa_attend current with
 *     one row written per token;
 *   - when p + 1 is a multiple of m: entry row (p + 1) / m - 1 of `entries` = the pooling of the
 *     m staged rows of the block, bitwise the entry csa_compress builds from the same rows
 *     (e[j,c] = sum_i softmax_i(g[i,c] + bias[i]) x[i,c], same arithmetic and order), stored by
 *     the same rules; not written outside [0, entries->rows).
 *   Indexer keys ([hongke] 4.1: a cache of their own; reading: pooled like the rows they index):
 *     a second call with x_new = the token's indexer key, g_new = its gate logits, d_c = d_I,
 *     d_r = 0, raw = NULL, and an E4M3 key store as `entries` keeps the csa_index key cache
 *     (scale = its sigma_k) in step.
 *   x_new, g_new [B][d] in in_dtype (F32 or BF16), d = d_c + d_r <= 1024. bias [m] fp32.
 *   stage_x, stage_g [B][m][d] fp32: caller-owned staging ring, kept between calls (the rows of
 *     earlier positions of the open block must hold those tokens). Store rows are per sequence
 *     (batch stride rows); the raw store is the window store csa_attend reads with pos0 = raw_pos0.
 *   Errors: CSA_EINVAL for a bad dtype, m <= 0, B < 0, non-positive d_c, NULL arguments (other
 *     than raw, raw_pos0) or store fields inconsistent with d_c / d_r / dtype; CSA_EUNSUPPORTED
 *     for d > 1024.
 * ------------------------------------------------------------------------------------------- */
csa_status csa_cache_append(const void* x_new, const void* g_new, int32_t in_dtype,
                            const float* bias, int32_t m, int32_t B, const int64_t* pos,
                            int32_t d_c, int32_t d_r, float* stage_x, float* stage_g,
                            const csa_kv_out_t* entries, const csa_kv_out_t* raw,
                            const int64_t* raw_pos0, void* stream);

/* ---------------------------------------------------------------------------------------------
 * csa_index -- lightning-indexer scores of every visible entry for every query.
 * [csdn] V4 改进一 and [yudong] 2.2 Step 2 (a light indexer, in the manner of the V3.2 lightning
 * indexer, scores each compressed row against the query; fp8 accelerated).
 *   s[i][j] = sum_h w[i][h] * max(0, qI[i][h] . kI[seq[i]][j])  for j < n_vis(pos[i]).
 *   q_i    [nq][H_I][d_I] in qi_dtype (F32, BF16 or E4M3); q_i_scale [nq][H_I] fp32 iff E4M3.
 *   w      [nq][H_I] fp32 head weights (any sign).
 *   k_i    [B][N][d_I] in ki_dtype (same dtype as q_i); k_i_scale [B][N] fp32 iff E4M3.
 *          For fp8: qI = q_i_scale * q_i and kI = k_i_scale * k_i.
 *   scores [nq][ld_scores] fp32, ld_scores >= N. Columns j >= n_vis(pos[i]) are not written.
 *   Constraints: d_I == 64 for E4M3/BF16 fast paths; any d_I % 4 == 0 otherwise, with
 *   H_I * (d_I + 1) * 4 <= 32 KiB (CSA_EUNSUPPORTED otherwise).
 * ------------------------------------------------------------------------------------------- */
csa_status csa_index(const csa_queries_t* Q, const void* q_i, const float* q_i_scale,
                     int32_t qi_dtype, const float* w, int32_t H_I, int32_t d_I, const void* k_i,
                     const float* k_i_scale, int32_t ki_dtype, int32_t B, int64_t N, int32_t m,
                     float* scores, int64_t ld_scores, void* stream);

/* ---------------------------------------------------------------------------------------------
 * csa_index_mxfp4 -- the low-precision indexer: MXFP4 queries and keys, bf16 scores.
 * [csdn] V4 的其他升级 (FP4 paragraph: the indexer's QK path in FP4 with fine-grained scales, which
 * widen losslessly to FP8; index scores in BF16) and [jaylab] 其他技术细节 (FP4 for the indexer QK
 * path). Same score as csa_index: s[i][j] = sum_h w[i][h] * max(0, qI[i][h] . kI[seq[i]][j]) for
 * j < n_vis(pos[i]), stored as bf16 (round to nearest even of the fp32 value).
 *   MXFP4 vectors (OCP Microscaling): E2M1 codes, two per byte, element 2e in the low nibble of
 *   byte e; one E8M0 scale byte per 32 consecutive elements (value = E2M1 * 2^(scale - 127)).
 *   q_i  [nq][H_I][d_I / 2] codes, q_i_scale [nq][H_I][d_I / 32] scales.
 *   k_i  [B][N][d_I / 2] codes, k_i_scale [B][N][d_I / 32] scales.
 *   w    [nq][H_I] fp32 head weights.
 *   scores [nq][ld_scores] bf16 codes, ld_scores >= N; columns >= n_vis are not written.
 *   Constraints: H_I == 8, d_I == 64 (CSA_EUNSUPPORTED otherwise); q_i and k_i 16-byte aligned.
 *   Per-block dot products are exact (E2M1 products are exact); head sums fp32.
 * ------------------------------------------------------------------------------------------- */
csa_status csa_index_mxfp4(const csa_queries_t* Q, const uint8_t* q_i, const uint8_t* q_i_scale,
                           const float* w, int32_t H_I, int32_t d_I, const uint8_t* k_i,
                           const uint8_t* k_i_scale, int32_t B, int64_t N, int32_t m,
                           uint16_t* scores, int64_t ld_scores, void* stream);

/* ---------------------------------------------------------------------------------------------
 * csa_topk -- per-query selection of the k highest-scoring visible entries.
 * [csdn] V4 改进一 and [yudong] 2.2 Step 3 (top-k; the pages use k = 64 and k = 1024).
 *   Among j < n_vis(pos[i]), order by score descending then index ascending (ties go to the lower
 *   index); take the first min(k, n_vis); write them to idx[i][0..) in ascending index order and
 *   pad with -1. -0.0 and +0.0 compare equal. Scores must not be NaN.
 *   scores [nq][ld_scores] fp32 (columns >= n_vis are not read); idx [nq][k] int32.
 *   Rows longer than 32768 need k <= 2048 and ceil(N / 32768) * k <= 32768 (CSA_EUNSUPPORTED).
 *   Workspace: csa_topk_workspace_bytes(nq, N, k). Deterministic (integer work only).
 * ------------------------------------------------------------------------------------------- */
csa_status csa_topk(const csa_queries_t* Q, const float* scores, int64_t ld_scores, int64_t N,
                    int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);
size_t csa_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k);

/* csa_topk_noalloc -- csa_topk for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): same arguments, rule and
 * results as csa_topk, without (ws, ws_bytes). Its scratch is a device array inside the library,
 * 16 MiB per GPU, held by every GPU the library runs on until the process ends; the call
 * allocates nothing. Calls whose csa_topk_workspace_bytes(nq, N, k) exceeds 16 MiB fail with
 * CSA_EWORKSPACE (rows of up to 32768 entries need none). Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (several streams or host threads) race on it. Nothing in
 * it needs to start at zero: a call writes every slot it reads. */
csa_status csa_topk_noalloc(const csa_queries_t* Q, const float* scores, int64_t ld_scores,
                            int64_t N, int32_t m, int32_t k, int32_t* idx, void* stream);

/* csa_topk_bf16 -- csa_topk on bf16 scores (csa_index_mxfp4's output), same rule and workspace
 * ([csdn] V4 的其他升级: bf16 index scores make the selection faster). scores [nq][ld_scores] bf16
 * codes; ties (far more frequent at bf16's 8 significant bits) go to the lower index. */
csa_status csa_topk_bf16(const csa_queries_t* Q, const uint16_t* scores, int64_t ld_scores,
                         int64_t N, int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                         void* stream);

/* ---------------------------------------------------------------------------------------------
 * csa_attend -- CSA attention: the selected entries plus the raw sliding window, one softmax.
 * [csdn] V4 改进一 (MQA with one KV shared by all heads; a short window of the most recent raw KV
 * bypasses compression) and [yudong] 2.2 Step 4; [csdn] MLA (key row [c; r], value row c).
 *   Keys of query i: entries idx[i][0..k) (entries of sequence seq[i]; -1 slots skipped), then raw
 *   rows for positions max(0, pos - window + 1) .. pos (no de-duplication). For head h:
 *     l = sm_scale * (q[i][h][:d_c] . c_key + q[i][h][d_c:] . r_key),  p = softmax(l),
 *     out[i][h] = sum p * c_key,  lse[i][h] = log sum exp(l)   (natural log).
 *   An empty key set gives out = 0, lse = -inf.
 *   q      [nq][H][d_c + d_r] in q_dtype (CSA_F32 with F32 stores, else CSA_BF16).
 *   entries, raw  stores with identical dtype_c, d_c, d_r; raw (a ring, see csa_kv_t) must hold
 *          every window position of every query: positions pos - window + 1 .. pos must be among
 *          the last raw->rows positions written to it. Selected slots holding a row at or past
 *          entries->rows are skipped like -1 slots.
 *   out    [nq][H][d_c] fp32; lse [nq][H] fp32 (may be NULL).
 *   Shapes: d_c <= 1024, d_c + d_r even and <= 4096 (else CSA_EUNSUPPORTED; the same for
 *   csa_attend_tokens and hca_attend).
 *   Workspace: csa_attend_workspace_bytes(nq, H, d_c, k + window).
 * ------------------------------------------------------------------------------------------- */
csa_status csa_attend(const csa_queries_t* Q, const void* q, int32_t q_dtype, int32_t H,
                      const csa_kv_t* entries, int32_t m, const int32_t* idx, int32_t k,
                      const csa_kv_t* raw, int32_t window, float sm_scale, float* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream);
size_t csa_attend_workspace_bytes(int32_t nq, int32_t H, int32_t d_c, int64_t max_keys);

/* ---------------------------------------------------------------------------------------------
 * csa_attend_tokens -- CSA attention over the original tokens of the selected blocks plus the
 * raw window, one softmax (the token-selection variant).
 * [hongke] 2.2 (item 3: fine-grained attention over the original tokens of each retrieved block)
 * and [yudong] 2.2 Steps 3-4 (the top-1024 blocks stand for 4096 original tokens, attended in
 * full); [csdn] V4 改进一 for the window and the MQA form.
 *   Keys of query i: for each slot s of idx[i][0..k) holding a block j >= 0 (-1 slots skipped),
 *   the raw rows of positions j*m .. j*m + m - 1 in that order; then the window positions
 *   max(0, pos - window + 1) .. pos (no de-duplication). Logits, softmax, out and lse as in
 *   csa_attend (K = [c; r], V = c).
 *   raw    the store of raw token rows (dtype_c BF16 or E4M3 with scale; F32 with F32 q). Token
 *          rows are read at row p - pos0[seq]: the store must hold every position of the selected
 *          blocks and of the window without wrapping (rows > every such p - pos0); a token row
 *          outside [0, rows) is skipped. The window follows the ring rule of csa_kv_t.
 *   idx    [nq][k] int32 block indices of the m-fold compression (csa_topk's output).
 *   Workspace: csa_attend_workspace_bytes(nq, H, d_c, k * m + window).
 *   Errors: as csa_attend; CSA_EINVAL also when k * m + window exceeds 2^30.
 * ------------------------------------------------------------------------------------------- */
csa_status csa_attend_tokens(const csa_queries_t* Q, const void* q, int32_t q_dtype, int32_t H,
                             const csa_kv_t* raw, int32_t m, const int32_t* idx, int32_t k,
                             int32_t window, float sm_scale, float* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * hca_attend -- HCA attention: dense attention over every visible m'-compressed entry.
 * [csdn] V4 改进一 (HCA) and [yudong] 2.3 Step 2: no selection and no window.
 *   Keys of query i: entries j < n_vis(pos[i]) of sequence seq[i] with m = m_prime; otherwise as
 *   csa_attend. Workspace: hca_attend_workspace_bytes(nq, H, d_c, N).
 * ------------------------------------------------------------------------------------------- */
csa_status hca_attend(const csa_queries_t* Q, const void* q, int32_t q_dtype, int32_t H,
                      const csa_kv_t* entries, int32_t m_prime, float sm_scale, float* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream);
size_t hca_attend_workspace_bytes(int32_t nq, int32_t H, int32_t d_c, int64_t N);

/* ---------------------------------------------------------------------------------------------
 * Instrumentation (not a step of the layer). Times the main attention kernel of csa_attend
 * (slot 0) and hca_attend (slot 1) alone, without the split-combine and fixup passes that follow
 * it, with a HIP event pair recorded on the caller's stream around that kernel.
 *   csa_kernel_timing_enable(cap): record the next cap launches per slot (0 <= cap <= 1024);
 *     cap = 0 stops recording and releases the events. Creates HIP events: call outside graph
 *     capture. The timing state is the library's one piece of mutable state: it is guarded by a
 *     mutex, and while timing is off an attention call only reads an atomic flag. Launches from
 *     several host threads while timing is on are recorded in the order they take the lock.
 *   csa_kernel_timing_read(slot, &ms, &n): waits for the recorded launches of the slot, returns
 *     their total duration in milliseconds and their count, and clears the slot.
 *   Errors: CSA_EINVAL for a capacity or slot out of range or NULL outputs; CSA_EHIP otherwise.
 * ------------------------------------------------------------------------------------------- */
csa_status csa_kernel_timing_enable(int32_t cap);
csa_status csa_kernel_timing_read(int32_t slot, double* ms, int32_t* n);

/* ---------------------------------------------------------------------------------------------
 * Instrumentation (not a step of the layer): the device's measured dense bf16 matrix-core rate,
 * the denominator beside the datasheet peak when a kernel is rated against the MFMA roofline.
 *   csa_peak_mfma_bf16(iters, sink, &tflops, stream): launches 768 blocks of 4 waves (3 per CU),
 *     each wave running 4 independent chains of iters mfma_f32_32x32x16_bf16 on register operands
 *     (no memory traffic in the loop), once short to warm up and once timed with a HIP event pair
 *     on `stream`; waits for it and returns the rate in TFLOP/s. sink: device memory of at least
 *     csa_peak_sink_floats() floats, owned by the caller, overwritten with one sum per wave.
 *     Creates HIP events: call outside graph capture.
 *   Errors: CSA_EINVAL for iters <= 0 or NULL sink / tflops; CSA_EHIP otherwise.
 * ------------------------------------------------------------------------------------------- */
csa_status csa_peak_mfma_bf16(int32_t iters, float* sink, double* tflops, void* stream);
int32_t csa_peak_sink_floats(void);

/* Text of a status code; for CSA_EHIP the text of the last HIP error seen by this thread. */
const char* csa_status_str(int32_t status);
const char* csa_last_error(void);
int32_t csa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
