// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once
#include <hip/hip_runtime.h>

#include "csa_mi355x.h"
#include <stddef.h>
#include <stdint.h>

namespace csa {

// Brackets one kernel launch with hipEvents when launch timing is enabled
// (csa_profile_enable); a no-op otherwise.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t st);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  hipStream_t st_;
  long idx_;
};

// Sets the calling thread's error text (csa_last_error) and returns st.
csa_status_t set_error(csa_status_t st, const char* fmt, ...);

// Raises a kernel's dynamic LDS limit to `lds` bytes (needed above 64 KiB)
// once per (device, kernel); thread-safe.
hipError_t ensure_lds_limit(const void* kfn, size_t lds);

// Device event counters (measurement only), read by csa_profile_counter.
enum CounterId { CNT_PREFILL_FALLBACK = 0, CNT_DECODE_FALLBACK = 1, CNT_STEP_TIMEOUT = 2,
                 CNT_DECODE_SECOND_ROUND = 3, CNT_COUNT = 4 };
hipError_t counter_read(int which, unsigned long long* value, bool reset);
// Device address of the counters (this device), for kernels in other
// translation units.
hipError_t counters_device_ptr(unsigned long long** p);

struct CompressArgs {
  const void *k, *v, *ki;
  const float *gate, *pos_bias;
  int B, T, d, dI, m, width, Nc_cap;   // width: tokens pooled per entry (m: no overlap)
  bool f32;
  void *kc, *vc, *kic;
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t st);

enum QkType { QK_F32 = 0, QK_BF16 = 1, QK_FP8 = 2, QK_FP4 = 3 };

struct IndexerArgs {
  const void *qi, *qi_scale;
  const float* w;
  const void *kic, *kic_scale;
  const int32_t* pos0;
  int max_pos;
  int B, Tq, Nc_cap, HI, dI, m, topk;
  QkType qk;
  int32_t* idx_out;
  float* score_out;
  void* ws;
};
size_t indexer_workspace(int B, int Tq, int Nc_cap, int HI, int dI, int topk, int qk);
hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t st);
// Decode rows long enough for the chunked path (score kernel + per-row pick):
// whether `a` takes it, and its score kernel alone (the pick left to the caller).
bool indexer_long_path(const IndexerArgs& a);
hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t st);

struct AttendArgs {
  bool sparse;                     // CSA (idx list) or HCA (dense over completed blocks)
  const void *q, *kc, *vc;
  const int32_t* idx;
  int topk;
  int m_prime;                     // HCA block size
  const void *kw, *vw;
  const int32_t* raw_pos0;
  int R, window;
  const int32_t* pos0;
  int max_pos;
  const float* sink;
  float scale;
  int B, Tq, H, d, Nc_cap;
  bool f32;
  void* out;
  float* lse;
  void* ws;
  // FP8 cache storage (kv8): K rows hold d/2 E4M3 codes (dims 0..d/2-1, one
  // fp32 scale per row) and d/2 bf16 values (dims d/2..d-1, the RoPE part); V
  // rows hold d codes with one fp32 scale per row.  kc/vc are unused then.
  bool kv8;
  const void *k8, *krope, *v8;
  const float *kscale, *vscale;
};
size_t attend_workspace(bool sparse, int B, int Tq, int H, int d, int topk, int window,
                        int Nc_cap, int m_prime, int max_pos);
hipError_t launch_attend(const AttendArgs& a, hipStream_t st);
// Both attention problems of a hybrid layer pair (csa_a sparse, hca_a dense),
// in one launch (plus one merge launch) when their split-decode kernels share a shape.
hipError_t launch_attend_pair(const AttendArgs& csa_a, const AttendArgs& hca_a, hipStream_t st);

struct ProjArgs {
  const void *o, *w;
  void* y;
  int T, G, K, dg;                 // tokens, groups, inputs per group ((H/G) d), outputs per group
  bool f32;
};
hipError_t launch_proj(const ProjArgs& a, hipStream_t st);

}  // namespace csa
