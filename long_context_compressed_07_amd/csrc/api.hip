// extern "C" entry points of libcsa (declared in include/csa.h): host-side validation of scalars,
// pointers and shapes, then dispatch to the kernel launchers. Nothing is enqueued on error.
#include <string>

#include "append.h"
#include "csa_internal.h"

namespace {

thread_local std::string g_last_error;

csa_status fail(csa_status s, const char* what) {
  g_last_error = what;
  return s;
}

csa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return CSA_OK;
  g_last_error = hipGetErrorString(e);
  return CSA_EHIP;
}

bool valid_dtype(int32_t d) { return d == CSA_F32 || d == CSA_BF16 || d == CSA_E4M3; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

csa::Store to_store(const csa_kv_t& k) {
  return csa::Store{k.c, k.r, k.scale, k.pos0, k.dtype_c, k.d_c, k.d_r, k.rows, k.ld_c, k.ld_r};
}

// Shape and pointer checks common to every cache-row store.
csa_status check_store(const csa_kv_t* s, const char* name) {
  static thread_local std::string msg;
  msg = std::string(name);
  if (s == nullptr) return fail(CSA_EINVAL, (msg + ": null store").c_str());
  if (!valid_dtype(s->dtype_c)) return fail(CSA_EINVAL, (msg + ": bad dtype_c").c_str());
  if (s->d_c <= 0 || s->d_r < 0 || s->rows < 0) return fail(CSA_EINVAL, (msg + ": bad dims").c_str());
  if (s->ld_c < s->d_c || (s->d_r > 0 && s->ld_r < s->d_r))
    return fail(CSA_EINVAL, (msg + ": leading dimension below row width").c_str());
  if (s->rows > 0 && s->c == nullptr) return fail(CSA_EINVAL, (msg + ": null c").c_str());
  if ((s->d_r > 0) != (s->r != nullptr)) return fail(CSA_EINVAL, (msg + ": r must be set iff d_r > 0").c_str());
  if ((s->dtype_c == CSA_E4M3) != (s->scale != nullptr))
    return fail(CSA_EINVAL, (msg + ": scale must be set iff dtype_c is E4M3").c_str());
  return CSA_OK;
}

csa_status check_queries(const csa_queries_t* Q) {
  if (Q == nullptr) return fail(CSA_EINVAL, "null queries");
  if (Q->nq < 0) return fail(CSA_EINVAL, "nq < 0");
  if (Q->nq > 0 && (Q->seq == nullptr || Q->pos == nullptr))
    return fail(CSA_EINVAL, "null query seq/pos");
  return CSA_OK;
}

}  // namespace

namespace csa {
// Measured dense bf16 MFMA rate (peak.hip): synchronises with the stream; sink holds
// peak_sink_floats() floats of device memory.
int peak_sink_floats();
hipError_t peak_mfma_bf16(int iters, float* sink, double* tflops, hipStream_t s);
}  // namespace csa

extern "C" {

int32_t csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return g_last_error.c_str(); }

const char* csa_status_str(int32_t status) {
  switch (status) {
    case CSA_OK: return "ok";
    case CSA_EINVAL: return "invalid argument";
    case CSA_EUNSUPPORTED: return "unsupported dtype/shape combination";
    case CSA_EWORKSPACE: return "workspace too small";
    case CSA_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

csa_status csa_compress(const void* x, const void* g, int32_t in_dtype, const float* bias,
                        int32_t m, int32_t B, int64_t T, int32_t d_c, int32_t d_r,
                        const float* hidden, const float* w_x, const float* w_g, int32_t d_model,
                        const csa_kv_out_t* out, float* raw_x_out, void* stream) {
  if (bias == nullptr || out == nullptr) return fail(CSA_EINVAL, "null bias or out");
  if (m < 1 || B < 0 || T < 0 || d_c <= 0 || d_r < 0) return fail(CSA_EINVAL, "bad sizes");
  if (in_dtype != CSA_F32 && in_dtype != CSA_BF16) return fail(CSA_EINVAL, "in_dtype must be F32 or BF16");
  if (!valid_dtype(out->dtype_c)) return fail(CSA_EINVAL, "bad out dtype");
  if (out->d_c != d_c || out->d_r != d_r) return fail(CSA_EINVAL, "out dims differ from d_c/d_r");
  if (out->rows != T / m) return fail(CSA_EINVAL, "out->rows must equal T / m");
  if (out->ld_c < d_c || (d_r > 0 && out->ld_r < d_r)) return fail(CSA_EINVAL, "out leading dimension");
  if ((B > 0 && out->rows > 0) && out->c == nullptr) return fail(CSA_EINVAL, "null out->c");
  if ((d_r > 0) != (out->r != nullptr)) return fail(CSA_EINVAL, "out->r must be set iff d_r > 0");
  if ((out->dtype_c == CSA_E4M3) != (out->scale != nullptr))
    return fail(CSA_EINVAL, "out->scale must be set iff out dtype is E4M3");
  const int d = d_c + d_r;
  const bool proj = hidden != nullptr || w_x != nullptr || w_g != nullptr || raw_x_out != nullptr;
  if (proj) {
    if (x != nullptr || g != nullptr) return fail(CSA_EINVAL, "projection mode takes no x/g");
    if (!hidden || !w_x || !w_g || !raw_x_out) return fail(CSA_EINVAL, "projection mode needs hidden, w_x, w_g, raw_x_out");
    if (in_dtype != CSA_F32 || d_model <= 0) return fail(CSA_EINVAL, "projection mode is fp32 with d_model > 0");
    if (d % 64 != 0 || d_c % 2 != 0 || d_model % 4 != 0 || (m != 1 && m != 2 && m != 4) ||
        out->dtype_c == CSA_E4M3)
      return fail(CSA_EUNSUPPORTED,
                  "projection mode needs d % 64 == 0, even d_c, d_model % 4 == 0, m in {1,2,4}, non-fp8 out");
    if (!aligned16(hidden) || !aligned16(w_x) || !aligned16(w_g))
      return fail(CSA_EUNSUPPORTED, "projection operands must be 16-byte aligned");
  } else {
    if (B > 0 && T > 0 && (x == nullptr || g == nullptr)) return fail(CSA_EINVAL, "null x or g");
    const int vec = in_dtype == CSA_F32 ? 4 : 8;
    if (d % vec != 0 || d_c % vec != 0 || d / vec > 256)
      return fail(CSA_EUNSUPPORTED, "d and d_c must be multiples of 16 bytes, d <= 256 vectors");
    if (!aligned16(x) || !aligned16(g)) return fail(CSA_EUNSUPPORTED, "x and g must be 16-byte aligned");
  }
  if (B == 0) return CSA_OK;
  csa::CompressArgs a{x, g, in_dtype, bias, m, B, T, d_c, d_r, hidden, w_x, w_g, d_model,
                      csa::OutStore{out->c, out->r, out->scale, out->dtype_c, out->d_c, out->d_r,
                                    out->rows, out->ld_c, out->ld_r},
                      raw_x_out};
  return hip_status(csa::launch_compress(a, static_cast<hipStream_t>(stream)));
}

csa_status csa_index(const csa_queries_t* Q, const void* q_i, const float* q_i_scale,
                     int32_t qi_dtype, const float* w, int32_t H_I, int32_t d_I, const void* k_i,
                     const float* k_i_scale, int32_t ki_dtype, int32_t B, int64_t N, int32_t m,
                     float* scores, int64_t ld_scores, void* stream) {
  if (csa_status st = check_queries(Q)) return st;
  if (!valid_dtype(qi_dtype) || qi_dtype != ki_dtype) return fail(CSA_EINVAL, "q_i and k_i must share a valid dtype");
  if (H_I <= 0 || d_I <= 0 || B <= 0 || N < 0 || m < 1 || ld_scores < N) return fail(CSA_EINVAL, "bad sizes");
  if (Q->nq > 0 && (q_i == nullptr || w == nullptr || scores == nullptr)) return fail(CSA_EINVAL, "null q_i/w/scores");
  if (N > 0 && k_i == nullptr) return fail(CSA_EINVAL, "null k_i");
  if (qi_dtype == CSA_E4M3 && (q_i_scale == nullptr || k_i_scale == nullptr))
    return fail(CSA_EINVAL, "fp8 indexer needs q_i_scale and k_i_scale");
  if ((size_t)H_I * (d_I + 1) * sizeof(float) > 32 * 1024) return fail(CSA_EUNSUPPORTED, "H_I * d_I too large");
  csa::IndexArgs a{csa::Queries{Q->seq, Q->pos, Q->nq}, q_i, q_i_scale, qi_dtype, w, H_I, d_I,
                   k_i, k_i_scale, B, N, m, scores, ld_scores};
  return hip_status(csa::launch_index(a, static_cast<hipStream_t>(stream)));
}

size_t csa_topk_workspace_bytes(int32_t nq, int64_t N, int32_t k) {
  return csa::topk_workspace(nq, N, k);
}

csa_status csa_topk(const csa_queries_t* Q, const float* scores, int64_t ld_scores, int64_t N,
                    int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (csa_status st = check_queries(Q)) return st;
  if (k < 1 || N < 0 || m < 1 || ld_scores < N) return fail(CSA_EINVAL, "bad sizes");
  if (Q->nq > 0 && (scores == nullptr || idx == nullptr)) return fail(CSA_EINVAL, "null scores/idx");
  if (!csa::topk_supported(N, k))
    return fail(CSA_EUNSUPPORTED,
                "rows longer than 32768 need k <= 2048 and ceil(N / 32768) * k <= 32768");
  const size_t need = csa::topk_workspace(Q->nq, N, k);
  if (ws_bytes < need || (need > 0 && ws == nullptr)) return fail(CSA_EWORKSPACE, "workspace too small");
  csa::TopkArgs a{csa::Queries{Q->seq, Q->pos, Q->nq}, scores, 0, ld_scores, N, m, k, idx, ws,
                  ws_bytes};
  return hip_status(csa::launch_topk(a, static_cast<hipStream_t>(stream)));
}

csa_status csa_topk_noalloc(const csa_queries_t* Q, const float* scores, int64_t ld_scores,
                            int64_t N, int32_t m, int32_t k, int32_t* idx, void* stream) {
  if (csa_status st = check_queries(Q)) return st;
  if (k < 1 || N < 0 || m < 1 || ld_scores < N) return fail(CSA_EINVAL, "bad sizes");
  if (Q->nq > 0 && (scores == nullptr || idx == nullptr)) return fail(CSA_EINVAL, "null scores/idx");
  if (!csa::topk_supported(N, k))
    return fail(CSA_EUNSUPPORTED,
                "rows longer than 32768 need k <= 2048 and ceil(N / 32768) * k <= 32768");
  const size_t need = csa::topk_workspace(Q->nq, N, k);
  if (need > csa::kTopkScratchBytes)
    return fail(CSA_EWORKSPACE, ("the call needs " + std::to_string(need) +
                                 " bytes of scratch; the no-allocation top-k holds " +
                                 std::to_string(csa::kTopkScratchBytes)).c_str());
  void* ws = nullptr;
  if (need > 0) {
    if (csa_status st = hip_status(csa::topk_scratch(&ws))) return st;
  }
  csa::TopkArgs a{csa::Queries{Q->seq, Q->pos, Q->nq}, scores, 0, ld_scores, N, m, k, idx, ws,
                  need};
  return hip_status(csa::launch_topk(a, static_cast<hipStream_t>(stream)));
}

csa_status csa_topk_bf16(const csa_queries_t* Q, const uint16_t* scores, int64_t ld_scores,
                         int64_t N, int32_t m, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                         void* stream) {
  if (csa_status st = check_queries(Q)) return st;
  if (k < 1 || N < 0 || m < 1 || ld_scores < N) return fail(CSA_EINVAL, "bad sizes");
  if (Q->nq > 0 && (scores == nullptr || idx == nullptr)) return fail(CSA_EINVAL, "null scores/idx");
  if (!csa::topk_supported(N, k))
    return fail(CSA_EUNSUPPORTED,
                "rows longer than 32768 need k <= 2048 and ceil(N / 32768) * k <= 32768");
  const size_t need = csa::topk_workspace(Q->nq, N, k);
  if (ws_bytes < need || (need > 0 && ws == nullptr)) return fail(CSA_EWORKSPACE, "workspace too small");
  csa::TopkArgs a{csa::Queries{Q->seq, Q->pos, Q->nq}, scores, 1, ld_scores, N, m, k, idx, ws,
                  ws_bytes};
  return hip_status(csa::launch_topk(a, static_cast<hipStream_t>(stream)));
}

csa_status csa_index_mxfp4(const csa_queries_t* Q, const uint8_t* q_i, const uint8_t* q_i_scale,
                           const float* w, int32_t H_I, int32_t d_I, const uint8_t* k_i,
                           const uint8_t* k_i_scale, int32_t B, int64_t N, int32_t m,
                           uint16_t* scores, int64_t ld_scores, void* stream) {
  if (csa_status st = check_queries(Q)) return st;
  if (B < 1 || N < 0 || m < 1 || ld_scores < N) return fail(CSA_EINVAL, "bad sizes");
  if (H_I != 8 || d_I != 64) return fail(CSA_EUNSUPPORTED, "the MXFP4 indexer takes 8 heads x 64");
  if (Q->nq > 0 && (q_i == nullptr || q_i_scale == nullptr || w == nullptr || scores == nullptr))
    return fail(CSA_EINVAL, "null query-side argument");
  if (N > 0 && (k_i == nullptr || k_i_scale == nullptr)) return fail(CSA_EINVAL, "null keys");
  if (((uintptr_t)q_i | (uintptr_t)k_i) & 15u) return fail(CSA_EINVAL, "q_i / k_i not 16-byte aligned");
  csa::IndexFp4Args a{csa::Queries{Q->seq, Q->pos, Q->nq}, q_i, q_i_scale, w, k_i, k_i_scale, B,
                      N, m, scores, ld_scores};
  return hip_status(csa::launch_index_fp4(a, static_cast<hipStream_t>(stream)));
}

size_t csa_attend_workspace_bytes(int32_t nq, int32_t H, int32_t d_c, int64_t max_keys) {
  return csa::attend_workspace(nq, H, d_c, max_keys, false);
}

size_t hca_attend_workspace_bytes(int32_t nq, int32_t H, int32_t d_c, int64_t N) {
  return csa::attend_workspace(nq, H, d_c, N, true);
}

namespace {

csa_status check_attend_common(const csa_queries_t* Q, const void* q, int32_t q_dtype, int32_t H,
                               const csa_kv_t* entries, int32_t m, float* out) {
  if (csa_status st = check_queries(Q)) return st;
  if (csa_status st = check_store(entries, "entries")) return st;
  if (q_dtype != CSA_F32 && q_dtype != CSA_BF16) return fail(CSA_EINVAL, "q_dtype must be F32 or BF16");
  if (H <= 0 || m < 1) return fail(CSA_EINVAL, "bad H or m");
  if (Q->nq > 0 && (q == nullptr || out == nullptr)) return fail(CSA_EINVAL, "null q or out");
  if (entries->d_c > 1024 || (entries->d_c + entries->d_r) % 2 != 0 ||
      entries->d_c + entries->d_r > 4096)
    return fail(CSA_EUNSUPPORTED, "d_c must be <= 1024, d_c + d_r even and <= 4096");
  return CSA_OK;
}

}  // namespace

csa_status csa_attend(const csa_queries_t* Q, const void* q, int32_t q_dtype, int32_t H,
                      const csa_kv_t* entries, int32_t m, const int32_t* idx, int32_t k,
                      const csa_kv_t* raw, int32_t window, float sm_scale, float* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (csa_status st = check_attend_common(Q, q, q_dtype, H, entries, m, out)) return st;
  if (k < 0 || window < 0) return fail(CSA_EINVAL, "negative k or window");
  if (k > 0 && Q->nq > 0 && idx == nullptr) return fail(CSA_EINVAL, "null idx");
  if (window > 0) {
    if (csa_status st = check_store(raw, "raw")) return st;
    if (raw->dtype_c != entries->dtype_c || raw->d_c != entries->d_c || raw->d_r != entries->d_r)
      return fail(CSA_EINVAL, "raw and entries stores differ in dtype or dims");
    if (raw->rows <= 0 && Q->nq > 0)
      return fail(CSA_EINVAL, "a window needs a raw store with rows > 0");
  }
  const size_t need = csa::attend_workspace(Q->nq, H, entries->d_c, (int64_t)k + window, false);
  if (ws_bytes < need || (need > 0 && ws == nullptr)) return fail(CSA_EWORKSPACE, "workspace too small");
  csa::AttendArgs a{};
  a.Q = csa::Queries{Q->seq, Q->pos, Q->nq};
  a.q = q;
  a.q_dtype = q_dtype;
  a.H = H;
  a.ent = to_store(*entries);
  a.m = m;
  a.dense = 0;
  a.idx = idx;
  a.k = k;
  if (window > 0) a.raw = to_store(*raw);
  a.window = window;
  a.sm_scale = sm_scale;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  return hip_status(csa::launch_attend(a, static_cast<hipStream_t>(stream)));
}

csa_status csa_attend_tokens(const csa_queries_t* Q, const void* q, int32_t q_dtype, int32_t H,
                             const csa_kv_t* raw, int32_t m, const int32_t* idx, int32_t k,
                             int32_t window, float sm_scale, float* out, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  if (csa_status st = check_attend_common(Q, q, q_dtype, H, raw, m, out)) return st;
  if (k < 0 || window < 0) return fail(CSA_EINVAL, "negative k or window");
  if (k > 0 && Q->nq > 0 && idx == nullptr) return fail(CSA_EINVAL, "null idx");
  if (raw->rows <= 0 && Q->nq > 0 && (k > 0 || window > 0))
    return fail(CSA_EINVAL, "token selection needs a raw store with rows > 0");
  if ((int64_t)k * m + window > (int64_t)1 << 30) return fail(CSA_EINVAL, "k * m + window too large");
  const size_t need = csa::attend_workspace(Q->nq, H, raw->d_c, (int64_t)k * m + window, false);
  if (ws_bytes < need || (need > 0 && ws == nullptr)) return fail(CSA_EWORKSPACE, "workspace too small");
  csa::AttendArgs a{};
  a.Q = csa::Queries{Q->seq, Q->pos, Q->nq};
  a.q = q;
  a.q_dtype = q_dtype;
  a.H = H;
  a.ent = to_store(*raw);    // unused by token selection (every key is a raw row)
  a.m = m;
  a.dense = 0;
  a.idx = idx;
  a.k = k;
  a.tok_m = m;
  a.raw = to_store(*raw);
  a.window = window;
  a.sm_scale = sm_scale;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  return hip_status(csa::launch_attend(a, static_cast<hipStream_t>(stream)));
}

csa_status hca_attend(const csa_queries_t* Q, const void* q, int32_t q_dtype, int32_t H,
                      const csa_kv_t* entries, int32_t m_prime, float sm_scale, float* out,
                      float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (csa_status st = check_attend_common(Q, q, q_dtype, H, entries, m_prime, out)) return st;
  const size_t need = csa::attend_workspace(Q->nq, H, entries->d_c, entries->rows, true);
  if (ws_bytes < need || (need > 0 && ws == nullptr)) return fail(CSA_EWORKSPACE, "workspace too small");
  csa::AttendArgs a{};
  a.Q = csa::Queries{Q->seq, Q->pos, Q->nq};
  a.q = q;
  a.q_dtype = q_dtype;
  a.H = H;
  a.ent = to_store(*entries);
  a.m = m_prime;
  a.dense = 1;
  a.idx = nullptr;
  a.k = 0;
  a.window = 0;
  a.sm_scale = sm_scale;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  return hip_status(csa::launch_attend(a, static_cast<hipStream_t>(stream)));
}

csa_status csa_kernel_timing_enable(int32_t cap) {
  if (cap < 0 || cap > csa::kTimingCap) return fail(CSA_EINVAL, "timing capacity out of range");
  return hip_status(csa::kernel_timing_enable(cap));
}

csa_status csa_cache_append(const void* x_new, const void* g_new, int32_t in_dtype,
                            const float* bias, int32_t m, int32_t B, const int64_t* pos,
                            int32_t d_c, int32_t d_r, float* stage_x, float* stage_g,
                            const csa_kv_out_t* entries, const csa_kv_out_t* raw,
                            const int64_t* raw_pos0, void* stream) {
  if (in_dtype != CSA_F32 && in_dtype != CSA_BF16) return fail(CSA_EINVAL, "in_dtype must be F32 or BF16");
  if (m <= 0 || B < 0 || d_c <= 0 || d_r < 0) return fail(CSA_EINVAL, "bad m / B / dims");
  if (d_c + d_r > 1024) return fail(CSA_EUNSUPPORTED, "d_c + d_r > 1024");
  if (B == 0) return CSA_OK;
  if (x_new == nullptr || g_new == nullptr || bias == nullptr || pos == nullptr ||
      stage_x == nullptr || stage_g == nullptr || entries == nullptr)
    return fail(CSA_EINVAL, "null argument");
  const csa_kv_out_t* st[2] = {entries, raw};
  for (const csa_kv_out_t* o : st) {
    if (o == nullptr) continue;   // no raw store
    if (!valid_dtype(o->dtype_c)) return fail(CSA_EINVAL, "bad store dtype");
    if (o->d_c != d_c || o->d_r != d_r) return fail(CSA_EINVAL, "store dims differ from d_c/d_r");
    if (o->rows < 0 || o->ld_c < d_c || (d_r > 0 && o->ld_r < d_r))
      return fail(CSA_EINVAL, "store rows / leading dimension");
    if (o->rows > 0 && o->c == nullptr) return fail(CSA_EINVAL, "null store c");
    if ((d_r > 0) != (o->r != nullptr)) return fail(CSA_EINVAL, "store r must be set iff d_r > 0");
    if ((o->dtype_c == CSA_E4M3) != (o->scale != nullptr))
      return fail(CSA_EINVAL, "store scale must be set iff its dtype is E4M3");
  }
  csa::AppendArgs a{};
  a.x_new = x_new;
  a.g_new = g_new;
  a.in_dtype = in_dtype;
  a.bias = bias;
  a.m = m;
  a.B = B;
  a.pos = pos;
  a.d_c = d_c;
  a.d_r = d_r;
  a.stage_x = stage_x;
  a.stage_g = stage_g;
  a.ent = csa::OutStore{entries->c, entries->r, entries->scale, entries->dtype_c, d_c, d_r,
                        entries->rows, entries->ld_c, entries->ld_r};
  if (raw != nullptr && raw->rows > 0)
    a.raw = csa::OutStore{raw->c, raw->r, raw->scale, raw->dtype_c, d_c, d_r, raw->rows,
                          raw->ld_c, raw->ld_r};
  a.raw_pos0 = raw_pos0;
  return hip_status(csa::launch_append(a, static_cast<hipStream_t>(stream)));
}

int32_t csa_peak_sink_floats(void) { return csa::peak_sink_floats(); }

csa_status csa_peak_mfma_bf16(int32_t iters, float* sink, double* tflops, void* stream) {
  if (iters <= 0 || sink == nullptr || tflops == nullptr) return fail(CSA_EINVAL, "bad peak query");
  return hip_status(csa::peak_mfma_bf16(iters, sink, tflops, static_cast<hipStream_t>(stream)));
}

csa_status csa_kernel_timing_read(int32_t slot, double* ms, int32_t* n) {
  if (ms == nullptr || n == nullptr || slot < 0 || slot > 1) return fail(CSA_EINVAL, "bad timing query");
  int cnt = 0;
  const csa_status st = hip_status(csa::kernel_timing_read(slot, ms, &cnt));
  *n = cnt;
  return st;
}

}  // extern "C"
