// C ABI of the CSA/HCA hot path: host-side validation, workspace sizing,
// thread-local error text, and dispatch to the gfx950 kernels.  Every entry
// point checks its arguments before touching the device; on any error it
// returns a status and launches nothing.
#include "csa_mi355x.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.hpp"
#include "step_tail.hpp"

namespace {

thread_local std::string g_err;

csa_status_t fail(csa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

csa_status_t ok() {
  g_err.clear();
  return CSA_OK;
}

csa_status_t device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSA_DEVICE_ERROR, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQUIRE(cond, st, ...)                 \
  do {                                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p, name)                                                        \
  do {                                                                              \
    REQUIRE((p) != nullptr, CSA_INVALID_ARGUMENT, "%s must not be NULL", name);     \
    REQUIRE(aligned((p), 16), CSA_INVALID_ARGUMENT, "%s must be 16-byte aligned", name); \
  } while (0)

#define REQUIRE_PTR4(p, name)                                                       \
  do {                                                                              \
    REQUIRE((p) != nullptr, CSA_INVALID_ARGUMENT, "%s must not be NULL", name);     \
    REQUIRE(aligned((p), 4), CSA_INVALID_ARGUMENT, "%s must be 4-byte aligned", name); \
  } while (0)

bool head_dim_ok(int d) { return d == 64 || d == 128; }
bool idx_dim_ok(int dI) { return dI == 32 || dI == 64; }
bool attn_dtype_ok(csa_dtype_t dt) { return dt == CSA_F32 || dt == CSA_BF16; }

// positions are int32: keep every derived count inside int range
constexpr long long kMaxElems = (long long)1 << 40;

}  // namespace

namespace csa {
csa_status_t set_error(csa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
}  // namespace csa

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return g_err.c_str(); }

csa_status_t csa_compress_window(const void* k, const void* v, const void* ki, const float* gate,
                                 const float* pos_bias, int B, int T, int d, int dI, int m,
                                 int width, int Nc_cap, csa_dtype_t dt, void* kc, void* vc,
                                 void* kic, void* stream) {
  REQUIRE(B >= 0 && T >= 0, CSA_INVALID_ARGUMENT, "B and T must be >= 0 (got %d, %d)", B, T);
  REQUIRE(m >= 1 && m <= 4096, CSA_INVALID_ARGUMENT, "m must be in [1, 4096] (got %d)", m);
  REQUIRE(width >= m && width <= 2 * m, CSA_INVALID_ARGUMENT,
          "width must be in [m, 2m] (got %d for m=%d)", width, m);
  REQUIRE(Nc_cap >= 0 && T / m <= Nc_cap, CSA_INVALID_ARGUMENT,
          "Nc_cap (%d) must hold T/m = %d entries", Nc_cap, T / m);
  REQUIRE(attn_dtype_ok(dt), CSA_UNSUPPORTED, "csa_compress: dtype must be CSA_F32 or CSA_BF16");
  REQUIRE(head_dim_ok(d), CSA_UNSUPPORTED, "head dim d=%d not built (64, 128)", d);
  REQUIRE((ki == nullptr) == (kic == nullptr), CSA_INVALID_ARGUMENT,
          "ki and kic must both be given or both be NULL");
  if (ki) REQUIRE(idx_dim_ok(dI), CSA_UNSUPPORTED, "indexer dim dI=%d not built (32, 64)", dI);
  REQUIRE((long long)B * T * d < kMaxElems, CSA_INVALID_ARGUMENT, "tensor too large");
  if (B == 0 || T / m == 0) return ok();
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(kc, "kc");
  REQUIRE_PTR(vc, "vc");
  REQUIRE_PTR4(gate, "gate");
  if (ki) {
    REQUIRE_PTR(ki, "ki");
    REQUIRE_PTR(kic, "kic");
  }
  if (pos_bias) REQUIRE(aligned(pos_bias, 4), CSA_INVALID_ARGUMENT, "pos_bias must be 4-byte aligned");
  csa::CompressArgs a{k, v, ki, gate, pos_bias, B, T, d, dI, m, width, Nc_cap, dt == CSA_F32, kc, vc, kic};
  return device_status(csa::launch_compress(a, (hipStream_t)stream), "csa_compress launch");
}

csa_status_t csa_compress(const void* k, const void* v, const void* ki, const float* gate,
                          const float* pos_bias, int B, int T, int d, int dI, int m, int Nc_cap,
                          csa_dtype_t dt, void* kc, void* vc, void* kic, void* stream) {
  return csa_compress_window(k, v, ki, gate, pos_bias, B, T, d, dI, m, m, Nc_cap, dt, kc, vc, kic,
                             stream);
}

size_t csa_indexer_topk_workspace(int B, int Tq, int Nc_cap, int HI, int dI, int topk,
                                  csa_dtype_t qk_dt) {
  if (B <= 0 || Tq <= 0 || Nc_cap <= 0) return 0;
  return csa::indexer_workspace(B, Tq, Nc_cap, HI, dI, topk, (int)qk_dt);
}

// Validation and argument packing shared by csa_indexer_topk and the decode step.
static csa_status_t build_indexer(const void* qi, const void* qi_scale, const float* w,
                                  const void* kic, const void* kic_scale, const int32_t* pos0,
                                  int max_pos, int B, int Tq, int Nc_cap, int HI, int dI, int m,
                                  int topk, csa_dtype_t qk_dt, int32_t* idx_out, float* score_out,
                                  void* workspace, size_t workspace_bytes, csa::IndexerArgs* a,
                                  bool* empty) {
  *empty = true;
  REQUIRE(B >= 0 && Tq >= 0, CSA_INVALID_ARGUMENT, "B and Tq must be >= 0");
  REQUIRE(Nc_cap >= 1, CSA_INVALID_ARGUMENT, "Nc_cap must be >= 1");
  REQUIRE(Nc_cap <= (1 << 23), CSA_UNSUPPORTED, "Nc_cap (%d) above 2^23 entries is not supported", Nc_cap);
  REQUIRE(m >= 1, CSA_INVALID_ARGUMENT, "m must be >= 1");
  REQUIRE(topk >= 1 && topk <= 4096, CSA_INVALID_ARGUMENT, "topk must be in [1, 4096] (got %d)", topk);
  REQUIRE(qk_dt == CSA_F32 || qk_dt == CSA_BF16 || qk_dt == CSA_FP8_E4M3 || qk_dt == CSA_FP4_E2M1,
          CSA_INVALID_ARGUMENT, "unknown qk dtype %d", (int)qk_dt);
  REQUIRE(HI == 1 || HI == 2 || HI == 4, CSA_UNSUPPORTED, "indexer heads HI=%d not built (1, 2, 4)", HI);
  REQUIRE(idx_dim_ok(dI), CSA_UNSUPPORTED, "indexer dim dI=%d not built (32, 64)", dI);
  REQUIRE(max_pos >= Tq - 1 && max_pos < INT_MAX / 2, CSA_INVALID_ARGUMENT,
          "max_pos (%d) must be >= Tq-1 and < 2^30", max_pos);
  REQUIRE((max_pos + 1) / m <= Nc_cap, CSA_INVALID_ARGUMENT,
          "the last query sees %d entries but Nc_cap is %d", (max_pos + 1) / m, Nc_cap);
  REQUIRE((long long)B * Tq * topk < kMaxElems && (long long)B * Nc_cap * dI < kMaxElems,
          CSA_INVALID_ARGUMENT, "tensor too large");
  if (B == 0 || Tq == 0) return ok();
  REQUIRE_PTR(qi, "qi");
  REQUIRE_PTR(kic, "kic");
  REQUIRE_PTR4(w, "w");
  REQUIRE_PTR4(pos0, "pos0");
  REQUIRE_PTR4(idx_out, "idx_out");
  if (score_out) REQUIRE(aligned(score_out, 4), CSA_INVALID_ARGUMENT, "score_out must be 4-byte aligned");
  if (qk_dt == CSA_FP8_E4M3) {
    REQUIRE_PTR4(qi_scale, "qi_scale");
    REQUIRE_PTR4(kic_scale, "kic_scale");
  } else if (qk_dt == CSA_FP4_E2M1) {
    REQUIRE(qi_scale && kic_scale, CSA_INVALID_ARGUMENT, "FP4 needs qi_scale and kic_scale");
  }
  const size_t need = csa_indexer_topk_workspace(B, Tq, Nc_cap, HI, dI, topk, qk_dt);
  REQUIRE(workspace_bytes >= need, CSA_WORKSPACE_TOO_SMALL,
          "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  if (need) REQUIRE_PTR(workspace, "workspace");
  *a = csa::IndexerArgs{qi, qi_scale, w, kic, kic_scale, pos0, max_pos, B, Tq, Nc_cap, HI, dI, m,
                        topk, (csa::QkType)qk_dt, idx_out, score_out, workspace};
  *empty = false;
  return ok();
}

csa_status_t csa_indexer_topk(const void* qi, const void* qi_scale, const float* w,
                              const void* kic, const void* kic_scale, const int32_t* pos0,
                              int max_pos, int B, int Tq, int Nc_cap, int HI, int dI, int m,
                              int topk, csa_dtype_t qk_dt, int32_t* idx_out, float* score_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  csa::IndexerArgs a;
  bool empty;
  const csa_status_t st = build_indexer(qi, qi_scale, w, kic, kic_scale, pos0, max_pos, B, Tq, Nc_cap,
                                        HI, dI, m, topk, qk_dt, idx_out, score_out, workspace,
                                        workspace_bytes, &a, &empty);
  if (st != CSA_OK || empty) return st;
  return device_status(csa::launch_indexer_topk(a, (hipStream_t)stream), "csa_indexer_topk launch");
}

size_t csa_sparse_attend_workspace(int B, int Tq, int H, int d, int topk, int window) {
  if (B <= 0 || Tq <= 0 || H <= 0) return 0;
  return csa::attend_workspace(true, B, Tq, H, d, topk, window, 1, 1, INT_MAX / 2);
}

size_t hca_attend_workspace(int B, int Tq, int H, int d, int Nc_cap, int m_prime, int window) {
  if (B <= 0 || Tq <= 0 || H <= 0 || m_prime <= 0) return 0;
  return csa::attend_workspace(false, B, Tq, H, d, 0, window, Nc_cap, m_prime, INT_MAX / 2);
}

static csa_status_t check_attend_common(const void* q, const void* kc, const void* vc,
                                        const void* kw, const void* vw, const int32_t* raw_pos0,
                                        int R, int window, const int32_t* pos0, int max_pos,
                                        const float* sink, int B, int Tq, int H, int d,
                                        int Nc_cap, csa_dtype_t dt, void* out, float* lse_out) {
  REQUIRE(B >= 0 && Tq >= 0, CSA_INVALID_ARGUMENT, "B and Tq must be >= 0");
  REQUIRE(H >= 1 && H <= 128, CSA_UNSUPPORTED, "query heads H=%d not supported (1..128)", H);
  REQUIRE(head_dim_ok(d), CSA_UNSUPPORTED, "head dim d=%d not built (64, 128)", d);
  REQUIRE(attn_dtype_ok(dt), CSA_UNSUPPORTED, "attention dtype must be CSA_F32 or CSA_BF16");
  REQUIRE(Nc_cap >= 1, CSA_INVALID_ARGUMENT, "Nc_cap must be >= 1");
  REQUIRE(window >= 0, CSA_INVALID_ARGUMENT, "window must be >= 0");
  REQUIRE(max_pos >= Tq - 1 && max_pos < INT_MAX / 2, CSA_INVALID_ARGUMENT,
          "max_pos (%d) must be >= Tq-1 and < 2^30", max_pos);
  REQUIRE((long long)B * Tq * H * d < kMaxElems && (long long)B * Nc_cap * d < kMaxElems,
          CSA_INVALID_ARGUMENT, "tensor too large");
  {
    // the kernels address one sequence's rows with 32-bit byte offsets
    const long long eb = dt == CSA_F32 ? 4 : 2;
    REQUIRE((long long)Tq * H * d * eb < (1LL << 31) && (long long)Nc_cap * d * eb < (1LL << 31) &&
                (window == 0 || (long long)R * d * eb < (1LL << 31)),
            CSA_INVALID_ARGUMENT, "one sequence's q, cache or raw rows exceed 2 GiB");
  }
  if (B == 0 || Tq == 0) return ok();
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(kc, "kc");
  REQUIRE_PTR(vc, "vc");
  REQUIRE_PTR(out, "out");
  REQUIRE_PTR4(pos0, "pos0");
  if (window > 0) {
    REQUIRE(R >= 1, CSA_INVALID_ARGUMENT, "window > 0 needs a raw buffer with R >= 1 rows");
    REQUIRE_PTR(kw, "kw");
    REQUIRE_PTR(vw, "vw");
    REQUIRE_PTR4(raw_pos0, "raw_pos0");
  }
  if (sink) REQUIRE(aligned(sink, 4), CSA_INVALID_ARGUMENT, "sink must be 4-byte aligned");
  if (lse_out) REQUIRE(aligned(lse_out, 4), CSA_INVALID_ARGUMENT, "lse_out must be 4-byte aligned");
  return ok();
}

// Validation and argument packing shared by csa_sparse_attend and
// csa_hybrid_attend; *empty is set when there is nothing to compute.
static csa_status_t build_sparse(const void* q, const void* kc, const void* vc, const int32_t* idx,
                                 int topk, const void* kw, const void* vw, const int32_t* raw_pos0,
                                 int R, const int32_t* pos0, int max_pos, int window,
                                 const float* sink, float softmax_scale, int B, int Tq, int H, int d,
                                 int Nc_cap, csa_dtype_t dt, void* out, float* lse_out,
                                 void* workspace, size_t workspace_bytes, csa::AttendArgs* a,
                                 bool* empty) {
  *empty = true;
  REQUIRE(topk >= 1 && topk <= 4096, CSA_INVALID_ARGUMENT, "topk must be in [1, 4096] (got %d)", topk);
  REQUIRE(softmax_scale > 0.f && softmax_scale < 1e30f, CSA_INVALID_ARGUMENT,
          "softmax_scale must be positive and finite (got %g)", (double)softmax_scale);
  csa_status_t st = check_attend_common(q, kc, vc, kw, vw, raw_pos0, R, window, pos0, max_pos,
                                        sink, B, Tq, H, d, Nc_cap, dt, out, lse_out);
  if (st != CSA_OK || B == 0 || Tq == 0) return st;
  REQUIRE_PTR4(idx, "idx");
  const size_t need = csa::attend_workspace(true, B, Tq, H, d, topk, window, Nc_cap, 1, max_pos);
  REQUIRE(workspace_bytes >= need, CSA_WORKSPACE_TOO_SMALL,
          "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  if (need) REQUIRE_PTR(workspace, "workspace");
  *a = csa::AttendArgs{};
  a->sparse = true; a->q = q; a->kc = kc; a->vc = vc; a->idx = idx; a->topk = topk; a->m_prime = 1;
  a->kw = window > 0 ? kw : nullptr; a->vw = window > 0 ? vw : nullptr;
  a->raw_pos0 = window > 0 ? raw_pos0 : nullptr; a->R = window > 0 ? R : 0; a->window = window;
  a->pos0 = pos0; a->max_pos = max_pos; a->sink = sink; a->scale = softmax_scale;
  a->B = B; a->Tq = Tq; a->H = H; a->d = d; a->Nc_cap = Nc_cap; a->f32 = dt == CSA_F32;
  a->out = out; a->lse = lse_out; a->ws = workspace;
  *empty = false;
  return ok();
}

csa_status_t csa_sparse_attend(const void* q, const void* kc, const void* vc, const int32_t* idx,
                               int topk, const void* kw, const void* vw, const int32_t* raw_pos0,
                               int R, const int32_t* pos0, int max_pos, int window,
                               const float* sink, float softmax_scale, int B, int Tq, int H, int d,
                               int Nc_cap, csa_dtype_t dt, void* out, float* lse_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  csa::AttendArgs a;
  bool empty;
  const csa_status_t st = build_sparse(q, kc, vc, idx, topk, kw, vw, raw_pos0, R, pos0, max_pos,
                                       window, sink, softmax_scale, B, Tq, H, d, Nc_cap, dt, out,
                                       lse_out, workspace, workspace_bytes, &a, &empty);
  if (st != CSA_OK || empty) return st;
  return device_status(csa::launch_attend(a, (hipStream_t)stream), "csa_sparse_attend launch");
}

static csa_status_t build_hca(const void* q, const void* kc, const void* vc, int m_prime, int Nc_cap,
                              const void* kw, const void* vw, const int32_t* raw_pos0, int R,
                              int window, const int32_t* pos0, int max_pos, const float* sink,
                              float softmax_scale, int B, int Tq, int H, int d, csa_dtype_t dt,
                              void* out, float* lse_out, void* workspace, size_t workspace_bytes,
                              csa::AttendArgs* a, bool* empty) {
  *empty = true;
  REQUIRE(m_prime >= 1, CSA_INVALID_ARGUMENT, "m_prime must be >= 1");
  REQUIRE(softmax_scale > 0.f && softmax_scale < 1e30f, CSA_INVALID_ARGUMENT,
          "softmax_scale must be positive and finite (got %g)", (double)softmax_scale);
  csa_status_t st = check_attend_common(q, kc, vc, kw, vw, raw_pos0, R, window, pos0, max_pos,
                                        sink, B, Tq, H, d, Nc_cap, dt, out, lse_out);
  if (st != CSA_OK || B == 0 || Tq == 0) return st;
  const size_t need = csa::attend_workspace(false, B, Tq, H, d, 0, window, Nc_cap, m_prime, max_pos);
  REQUIRE(workspace_bytes >= need, CSA_WORKSPACE_TOO_SMALL,
          "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  if (need) REQUIRE_PTR(workspace, "workspace");
  *a = csa::AttendArgs{};
  a->sparse = false; a->q = q; a->kc = kc; a->vc = vc; a->idx = nullptr; a->topk = 0; a->m_prime = m_prime;
  a->kw = window > 0 ? kw : nullptr; a->vw = window > 0 ? vw : nullptr;
  a->raw_pos0 = window > 0 ? raw_pos0 : nullptr; a->R = window > 0 ? R : 0; a->window = window;
  a->pos0 = pos0; a->max_pos = max_pos; a->sink = sink; a->scale = softmax_scale;
  a->B = B; a->Tq = Tq; a->H = H; a->d = d; a->Nc_cap = Nc_cap; a->f32 = dt == CSA_F32;
  a->out = out; a->lse = lse_out; a->ws = workspace;
  *empty = false;
  return ok();
}

csa_status_t hca_attend(const void* q, const void* kc, const void* vc, int m_prime, int Nc_cap,
                        const void* kw, const void* vw, const int32_t* raw_pos0, int R,
                        int window, const int32_t* pos0, int max_pos, const float* sink,
                        float softmax_scale, int B, int Tq, int H, int d, csa_dtype_t dt,
                        void* out, float* lse_out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  csa::AttendArgs a;
  bool empty;
  const csa_status_t st = build_hca(q, kc, vc, m_prime, Nc_cap, kw, vw, raw_pos0, R, window, pos0,
                                    max_pos, sink, softmax_scale, B, Tq, H, d, dt, out, lse_out,
                                    workspace, workspace_bytes, &a, &empty);
  if (st != CSA_OK || empty) return st;
  return device_status(csa::launch_attend(a, (hipStream_t)stream), "hca_attend launch");
}

// FP8 cache planes (validated after the shared checks, which see k8/v8 as kc/vc)
static csa_status_t add_kv8(csa::AttendArgs* a, int d, csa_dtype_t dt, const void* k8,
                            const void* krope, const float* kscale, const void* v8,
                            const float* vscale) {
  REQUIRE(dt == CSA_BF16, CSA_UNSUPPORTED, "FP8 caches need bf16 queries and window rows");
  REQUIRE(d == 128, CSA_UNSUPPORTED, "FP8 caches are built for d=128 (got %d)", d);
  REQUIRE_PTR(krope, "krope");
  REQUIRE_PTR4(kscale, "kscale");
  REQUIRE((v8 == nullptr) == (vscale == nullptr), CSA_INVALID_ARGUMENT,
          "v8 and vscale must both be given, or both be NULL (values = key rows)");
  if (vscale) REQUIRE_PTR4(vscale, "vscale");
  if (v8) REQUIRE_PTR(v8, "v8");
  a->kv8 = true;
  a->k8 = k8; a->krope = krope; a->v8 = v8; a->kscale = kscale; a->vscale = vscale;
  a->kc = nullptr; a->vc = nullptr;
  return ok();
}

csa_status_t csa_sparse_attend_kv8(const void* q, const void* k8, const void* krope,
                                   const float* kscale, const void* v8, const float* vscale,
                                   const int32_t* idx, int topk, const void* kw, const void* vw,
                                   const int32_t* raw_pos0, int R, const int32_t* pos0,
                                   int max_pos, int window, const float* sink, float softmax_scale,
                                   int B, int Tq, int H, int d, int Nc_cap, void* out,
                                   float* lse_out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  csa::AttendArgs a;
  bool empty;
  csa_status_t st = build_sparse(q, k8, v8 ? v8 : k8, idx, topk, kw, vw, raw_pos0, R, pos0, max_pos, window,
                                 sink, softmax_scale, B, Tq, H, d, Nc_cap, CSA_BF16, out, lse_out,
                                 workspace, workspace_bytes, &a, &empty);
  if (st != CSA_OK || empty) return st;
  st = add_kv8(&a, d, CSA_BF16, k8, krope, kscale, v8, vscale);
  if (st != CSA_OK) return st;
  return device_status(csa::launch_attend(a, (hipStream_t)stream), "csa_sparse_attend_kv8 launch");
}

csa_status_t hca_attend_kv8(const void* q, const void* k8, const void* krope, const float* kscale,
                            const void* v8, const float* vscale, int m_prime, int Nc_cap,
                            const void* kw, const void* vw, const int32_t* raw_pos0, int R,
                            int window, const int32_t* pos0, int max_pos, const float* sink,
                            float softmax_scale, int B, int Tq, int H, int d, void* out,
                            float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  csa::AttendArgs a;
  bool empty;
  csa_status_t st = build_hca(q, k8, v8 ? v8 : k8, m_prime, Nc_cap, kw, vw, raw_pos0, R, window, pos0, max_pos,
                              sink, softmax_scale, B, Tq, H, d, CSA_BF16, out, lse_out, workspace,
                              workspace_bytes, &a, &empty);
  if (st != CSA_OK || empty) return st;
  st = add_kv8(&a, d, CSA_BF16, k8, krope, kscale, v8, vscale);
  if (st != CSA_OK) return st;
  return device_status(csa::launch_attend(a, (hipStream_t)stream), "hca_attend_kv8 launch");
}

csa_status_t csa_hybrid_attend(
    const void* q, const void* kc, const void* vc, const int32_t* idx, int topk, const void* kw,
    const void* vw, const int32_t* raw_pos0, int R, const int32_t* pos0, int max_pos, int window,
    const float* sink, float softmax_scale, int B, int Tq, int H, int d, int Nc_cap, csa_dtype_t dt,
    void* out, float* lse_out, void* workspace, size_t workspace_bytes,
    const void* hq, const void* hkc, const void* hvc, int m_prime, int hNc_cap, const void* hkw,
    const void* hvw, const int32_t* hraw_pos0, int hR, int hwindow, const int32_t* hpos0,
    int hmax_pos, const float* hsink, float hsoftmax_scale, int hB, int hTq, int hH, int hd,
    csa_dtype_t hdt, void* hout, float* hlse_out, void* hworkspace, size_t hworkspace_bytes,
    void* stream) {
  csa::AttendArgs ac, ah;
  bool ec, eh;
  csa_status_t st = build_sparse(q, kc, vc, idx, topk, kw, vw, raw_pos0, R, pos0, max_pos, window,
                                 sink, softmax_scale, B, Tq, H, d, Nc_cap, dt, out, lse_out,
                                 workspace, workspace_bytes, &ac, &ec);
  if (st != CSA_OK) return fail(st, "CSA part: %s", g_err.c_str());
  st = build_hca(hq, hkc, hvc, m_prime, hNc_cap, hkw, hvw, hraw_pos0, hR, hwindow, hpos0, hmax_pos,
                 hsink, hsoftmax_scale, hB, hTq, hH, hd, hdt, hout, hlse_out, hworkspace,
                 hworkspace_bytes, &ah, &eh);
  if (st != CSA_OK) return fail(st, "HCA part: %s", g_err.c_str());
  if (!ec && !eh) {
    const size_t nc = csa::attend_workspace(true, B, Tq, H, d, topk, window, Nc_cap, 1, max_pos);
    const size_t nh = csa::attend_workspace(false, hB, hTq, hH, hd, 0, hwindow, hNc_cap, m_prime, hmax_pos);
    const uintptr_t c0 = (uintptr_t)workspace, h0 = (uintptr_t)hworkspace;
    REQUIRE(nc == 0 || nh == 0 || c0 + nc <= h0 || h0 + nh <= c0, CSA_INVALID_ARGUMENT,
            "the CSA and HCA workspaces overlap");
    REQUIRE(out != hout, CSA_INVALID_ARGUMENT, "the CSA and HCA outputs are the same buffer");
  }
  hipError_t e = hipSuccess;
  if (!ec && !eh) e = csa::launch_attend_pair(ac, ah, (hipStream_t)stream);
  else if (!ec) e = csa::launch_attend(ac, (hipStream_t)stream);
  else if (!eh) e = csa::launch_attend(ah, (hipStream_t)stream);
  return device_status(e, "csa_hybrid_attend launch");
}

// Workspace carve-up of the decode step: control words of the fused tail |
// indexer | CSA attention | HCA attention.
struct StepWs {
  size_t ctl, idx, csa, hca, total;
};
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static StepWs step_ws(const csa_decode_step_t* s) {
  StepWs w{};
  if (s->B <= 0) return w;
  const size_t ni = csa_indexer_topk_workspace(s->B, 1, s->Nc_cap, s->HI, s->dI, s->topk, s->qk_dt);
  const size_t nc = s->topk >= 1 ? csa::attend_workspace(true, s->B, 1, s->H, s->d, s->topk, s->window,
                                                         s->Nc_cap, 1, s->max_pos) : 0;
  const size_t nh = s->m_prime >= 1 ? csa::attend_workspace(false, s->B, 1, s->H, s->d, 0, s->hwindow,
                                                            s->hNc_cap, s->m_prime, s->max_pos) : 0;
  w.ctl = 0;
  w.idx = csa::decode_tail_ctl_bytes();
  w.csa = align256(w.idx + ni);
  w.hca = align256(w.csa + nc);
  w.total = w.hca + nh;
  return w;
}

size_t csa_hybrid_decode_step_workspace(const csa_decode_step_t* step) {
  if (step == nullptr || step->B <= 0 || step->H <= 0 || step->Nc_cap <= 0) return 0;
  return step_ws(step).total;
}

csa_status_t csa_hybrid_decode_step(const csa_decode_step_t* s, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  REQUIRE(s != nullptr, CSA_INVALID_ARGUMENT, "step must not be NULL");
  REQUIRE(s->B >= 0, CSA_INVALID_ARGUMENT, "B must be >= 0");
  REQUIRE((s->flags & ~(unsigned)CSA_STEP_FUSED_TAIL) == 0, CSA_INVALID_ARGUMENT,
          "flags holds undefined bits (0x%x)", s->flags);
  if (s->B == 0) return ok();
  REQUIRE(s->H >= 1 && s->Nc_cap >= 1 && s->m_prime >= 1 && s->topk >= 1, CSA_INVALID_ARGUMENT,
          "H, Nc_cap, m_prime and topk must be >= 1");
  REQUIRE(((uintptr_t)workspace % 256) == 0, CSA_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const StepWs wl = step_ws(s);
  REQUIRE(workspace_bytes >= wl.total, CSA_WORKSPACE_TOO_SMALL,
          "workspace holds %zu bytes, %zu needed", workspace_bytes, wl.total);
  if (wl.total) REQUIRE_PTR(workspace, "workspace");
  char* ws = reinterpret_cast<char*>(workspace);
  csa::IndexerArgs ai;
  csa::AttendArgs ac, ah;
  bool ei, ec, eh;
  csa_status_t st = build_indexer(s->qi, s->qi_scale, s->w, s->kic, s->kic_scale, s->pos0, s->max_pos,
                                  s->B, 1, s->Nc_cap, s->HI, s->dI, s->m, s->topk, s->qk_dt, s->idx_out,
                                  nullptr, ws ? ws + wl.idx : nullptr, wl.csa - wl.idx, &ai, &ei);
  if (st != CSA_OK) return fail(st, "indexer part: %s", g_err.c_str());
  st = build_sparse(s->q, s->kc, s->vc, s->idx_out, s->topk, s->kw, s->vw, s->raw_pos0, s->R, s->pos0,
                    s->max_pos, s->window, s->sink, s->softmax_scale, s->B, 1, s->H, s->d, s->Nc_cap,
                    s->dt, s->out, s->lse_out, ws ? ws + wl.csa : nullptr, wl.hca - wl.csa, &ac, &ec);
  if (st != CSA_OK) return fail(st, "CSA part: %s", g_err.c_str());
  st = build_hca(s->hq, s->hkc, s->hvc, s->m_prime, s->hNc_cap, s->hkw, s->hvw, s->hraw_pos0, s->hR,
                 s->hwindow, s->pos0, s->max_pos, s->hsink, s->hsoftmax_scale, s->B, 1, s->H, s->d, s->dt,
                 s->hout, s->hlse_out, ws ? ws + wl.hca : nullptr, wl.total - wl.hca, &ah, &eh);
  if (st != CSA_OK) return fail(st, "HCA part: %s", g_err.c_str());
  REQUIRE(s->out != s->hout, CSA_INVALID_ARGUMENT, "the CSA and HCA outputs are the same buffer");
  hipError_t e = hipSuccess;
  const bool fused = (s->flags & CSA_STEP_FUSED_TAIL) && !ei && !ec && !eh &&
                     csa::indexer_long_path(ai) && csa::decode_tail_supported(ac, ah);
  if (fused) {
    unsigned long long* counters = nullptr;
    e = csa::counters_device_ptr(&counters);
    // the row picks as their own 1024-thread launch (a 256-thread pick inside
    // the tail measured twice as long), then attention and merges in one launch
    if (e == hipSuccess) e = csa::launch_indexer_topk(ai, (hipStream_t)stream);
    if (e == hipSuccess)
      e = csa::launch_decode_tail(ai, ac, ah, ws + wl.ctl, counters, false, (hipStream_t)stream);
  } else {
    e = csa::launch_indexer_topk(ai, (hipStream_t)stream);
    if (e == hipSuccess) e = csa::launch_attend_pair(ac, ah, (hipStream_t)stream);
  }
  return device_status(e, "csa_hybrid_decode_step launch");
}

csa_status_t csa_grouped_out_proj(const void* o, const void* w, int T, int H, int d, int G, int dg,
                                  csa_dtype_t dt, void* y, void* stream) {
  REQUIRE(T >= 0, CSA_INVALID_ARGUMENT, "T must be >= 0");
  REQUIRE(H >= 1 && d >= 1 && G >= 1, CSA_INVALID_ARGUMENT, "H, d and G must be >= 1");
  REQUIRE(H % G == 0, CSA_INVALID_ARGUMENT, "G=%d must divide H=%d", G, H);
  const long long K = (long long)(H / G) * d;
  REQUIRE(K % 64 == 0, CSA_UNSUPPORTED, "inputs per group (H/G)*d = %lld must be a multiple of 64", K);
  REQUIRE(dg >= 128 && dg % 128 == 0, CSA_UNSUPPORTED, "outputs per group dg=%d must be a multiple of 128", dg);
  REQUIRE(attn_dtype_ok(dt), CSA_UNSUPPORTED, "dtype must be CSA_F32 or CSA_BF16");
  const long long eb = dt == CSA_F32 ? 4 : 2;
  REQUIRE((long long)T * H * d * eb < (1LL << 31), CSA_INVALID_ARGUMENT, "o exceeds 2 GiB");
  REQUIRE((long long)G * K * dg < kMaxElems && (long long)T * G * dg < kMaxElems, CSA_INVALID_ARGUMENT,
          "tensor too large");
  if (T == 0) return ok();
  REQUIRE_PTR(o, "o");
  REQUIRE_PTR(w, "w");
  REQUIRE_PTR(y, "y");
  csa::ProjArgs a{o, w, y, T, G, (int)K, dg, dt == CSA_F32};
  return device_status(csa::launch_proj(a, (hipStream_t)stream), "csa_grouped_out_proj launch");
}

}  // extern "C"
