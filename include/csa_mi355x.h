/*
 * csa_mi355x.h — C ABI of the CSA / HCA hybrid-attention hot path for AMD
 * Instinct MI355X (CDNA4, gfx950).
 *
 * The method (DeepSeek-V4 summaries: hyper.ai "Method", CSA and HCA
 * paragraphs; aiboss88 "Technical Principles", CSA / HCA / FP4 bullets):
 *   CSA  compresses every m tokens of the (single, MQA-shared) KV head into one
 *        entry, scores entries with a lightning indexer, keeps the top-k and
 *        attends over them plus a sliding window of raw tokens and a per-head
 *        attention sink.
 *   HCA  compresses every m' >> m tokens (no overlap) and attends densely over
 *        all completed entries (plus the sink and an optional window).
 * The pages give no equations; the forms implemented are:
 *   compress : a_i = k_i.g + b_(i mod m);  p = softmax over the block;
 *              Kc_j = sum p_i k_i, Vc_j = sum p_i v_i, KIc_j = sum p_i kI_i
 *   indexer  : I[t,j] = sum_h w[t,h] * max(0, qI[t,h].KIc_j),  j < floor((t+1)/m)
 *   top-k    : the k largest I[t,.], equal scores to the lower index,
 *              emitted ascending by index and padded with -1
 *   attention: one softmax over {selected entries} U {window tokens} U {sink}:
 *              o = sum e^(l-M) v / (e^(s_h-M) + sum e^(l-M)),  l = scale*q.key,
 *              lse = M + ln(denominator)
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library keeps no reference after the call returns and allocates no
 *     memory.  Scratch space is passed in as `workspace` (size from the
 *     matching *_workspace query; NULL allowed when that size is 0).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; nothing synchronises.
 *   - Arguments are validated on the host first.  On any error the call
 *     returns a non-zero status, launches nothing, writes nothing, and
 *     csa_last_error() describes the problem.
 *   - Tensors are dense and row-major in the shapes given; the batch stride
 *     of a cache is Nc_cap rows.  Every pointer must be 16-byte aligned.
 *   - Inputs must be finite; behaviour on NaN/Inf inputs is unspecified.
 *   - Index/position inputs that fall outside the stated bounds are clamped
 *     or skipped by the kernels (they never read or write out of bounds),
 *     but the result is then unspecified.
 */
#ifndef CSA_MI355X_H
#define CSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 1

typedef enum {
  CSA_OK = 0,
  CSA_INVALID_ARGUMENT = 1,    /* null/misaligned pointer, bad size, inconsistent shapes */
  CSA_UNSUPPORTED = 2,         /* valid but not built: head dim, dtype, head count ...  */
  CSA_WORKSPACE_TOO_SMALL = 3,
  CSA_DEVICE_ERROR = 4         /* a HIP call or kernel launch failed                    */
} csa_status_t;

typedef enum {
  CSA_F32 = 0,
  CSA_BF16 = 1,
  CSA_FP8_E4M3 = 2,            /* OCP E4M3 "fn" codes, one fp32 scale per row          */
  CSA_FP4_E2M1 = 3             /* OCP E2M1 codes, 2 per byte (even element in the low
                                  nibble), one E8M0 scale per 32 elements              */
} csa_dtype_t;

/* Returns CSA_ABI_VERSION of the built library. */
int csa_abi_version(void);

/* Text of the last error on the calling thread ("" if none).  Valid until the
 * next call into the library on the same thread. */
const char *csa_last_error(void);

/*
 * csa_compress — block compression (CSA with m, HCA with m').
 * hyper.ai "Method", CSA paragraph (m tokens -> one entry with learnable
 * compression weights and positional biases) and HCA paragraph (m' tokens,
 * non-overlapping).
 *
 *   k, v      [B, T, d]   raw keys / values of the one KV head (dt)
 *   ki        [B, T, dI]  raw indexer keys (dt), or NULL (then kic is NULL)
 *   gate      [d]  fp32   gate vector g;  a_i = k_i . g + pos_bias[i mod m]
 *   pos_bias  [m]  fp32   or NULL (= 0)
 *   kc, vc    [B, Nc_cap, d], kic [B, Nc_cap, dI]  outputs (dt); rows
 *             0 .. T/m - 1 are written (a trailing partial block is not).
 *   dt ∈ {CSA_F32, CSA_BF16}; d ∈ {64, 128}; dI ∈ {32, 64}; 1 <= m <= 4096;
 *   T/m <= Nc_cap.  Accumulation in fp32, bf16 outputs rounded to nearest even.
 */
csa_status_t csa_compress(const void *k, const void *v, const void *ki,
                          const float *gate, const float *pos_bias,
                          int B, int T, int d, int dI, int m, int Nc_cap, csa_dtype_t dt,
                          void *kc, void *vc, void *kic, void *stream);

/*
 * csa_compress_window — csa_compress with overlapping windows (CSA).
 * hyper.ai "Method": the HCA paragraph states that HCA compresses without
 * overlap, setting it apart from CSA, whose windows the page leaves open.
 * Entry j pools the `width` tokens ending where block j ends:
 *   rows t = (j+1)m - width + i, i = 0..width-1 (rows t < 0 are absent),
 *   a_i = k_t . g + pos_bias[i],  p = softmax over the window's rows,
 *   Kc_j = sum p_i k_t,  Vc_j = sum p_i v_t,  KIc_j = sum p_i kI_t.
 * m <= width <= 2m; width = m is csa_compress.  pos_bias has `width` entries
 * (window positions, oldest first) or is NULL.  Entry j is complete once
 * (j+1)m tokens exist, as without overlap; other arguments as csa_compress.
 */
csa_status_t csa_compress_window(const void *k, const void *v, const void *ki,
                                 const float *gate, const float *pos_bias,
                                 int B, int T, int d, int dI, int m, int width, int Nc_cap,
                                 csa_dtype_t dt, void *kc, void *vc, void *kic, void *stream);

/*
 * csa_indexer_topk — lightning-indexer scores and top-k selection.
 * hyper.ai "Method", CSA paragraph (a lightning indexer selects the top-k
 * compressed entries); aiboss88 "Technical Principles", CSA bullet (index
 * scores, top-k sparse selection) and FP4 bullet (FP4 indexer QK path, FP8
 * for dynamic range).
 *
 *   qi        [B, Tq, HI, dI]  indexer queries: F32/BF16 values, FP8 codes, or
 *             FP4 packed codes [B, Tq, HI, dI/2]
 *   qi_scale  NULL for F32/BF16; fp32 [B, Tq, HI] for FP8;
 *             uint8 E8M0 [B, Tq, HI, dI/32] for FP4
 *   w         [B, Tq, HI] fp32 per-token head weights (must be >= 0)
 *   kic       [B, Nc_cap, dI] compressed indexer keys (same encoding as qi;
 *             FP4: [B, Nc_cap, dI/2])
 *   kic_scale NULL / fp32 [B, Nc_cap] / uint8 E8M0 [B, Nc_cap, dI/32]
 *   pos0      [B] int32 device: query i of sequence b sits at absolute
 *             position pos0[b] + i and sees entries j < floor((pos+1)/m)
 *   max_pos   host upper bound of pos0[b] + Tq - 1 over b (validation: the
 *             last query may see at most Nc_cap entries)
 *   idx_out   [B, Tq, topk] int32: selected entries ascending, -1 padded when
 *             fewer than topk are eligible
 *   score_out [B, Tq, topk] fp32 scores aligned with idx_out (-inf where
 *             idx_out is -1), or NULL
 *   qk_dt ∈ {F32, BF16, FP8_E4M3, FP4_E2M1}; dI ∈ {32, 64}; HI ∈ {1, 2, 4};
 *   1 <= topk <= 4096; 1 <= Nc_cap <= 2^23.  FP8/FP4 codes are widened
 *   exactly to bf16 and scores accumulate in fp32; ReLU yields +0.
 */
size_t csa_indexer_topk_workspace(int B, int Tq, int Nc_cap, int HI, int dI, int topk,
                                  csa_dtype_t qk_dt);
csa_status_t csa_indexer_topk(const void *qi, const void *qi_scale, const float *w,
                              const void *kic, const void *kic_scale,
                              const int32_t *pos0, int max_pos,
                              int B, int Tq, int Nc_cap, int HI, int dI, int m, int topk,
                              csa_dtype_t qk_dt, int32_t *idx_out, float *score_out,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_sparse_attend — CSA core attention (MQA: H query heads, one KV head).
 * hyper.ai "Method", CSA paragraph (core attention over the selected entries,
 * MQA with shared keys and values) and HCA paragraph (sliding-window branch);
 * aiboss88 "Technical Principles", CSA bullet (sliding window + attention sink).
 *
 *   q, out    [B, Tq, H, d] (dt)
 *   kc, vc    [B, Nc_cap, d] compressed entries (dt)
 *   idx       [B, Tq, topk] int32 selected entries (-1 = unused slot)
 *   kw, vw    [B, R, d] raw tokens; row r holds absolute position
 *             raw_pos0[b] + r (prefill passes the whole sequence with
 *             raw_pos0 = 0, decode the last `window` tokens); NULL when
 *             window == 0
 *   raw_pos0  [B] int32 device (NULL when window == 0)
 *   pos0      [B] int32 device: query positions as for csa_indexer_topk
 *   window    W >= 0: the query at t also attends raw positions
 *             max(0, t-W+1) .. t (its own token included); window
 *             positions the raw buffer does not hold are left out, so
 *             queries at Tq positions need R >= W + Tq - 1 rows
 *   sink      [H] fp32 sink logits, or NULL for no sink
 *   lse_out   [B, Tq, H] fp32 natural-log denominators (incl. sink), or NULL
 *   softmax_scale  sigma > 0 (finite); logits are sigma * q.k
 *   dt ∈ {F32, BF16}; d ∈ {64, 128}; 1 <= H <= 128; topk <= 4096.
 */
size_t csa_sparse_attend_workspace(int B, int Tq, int H, int d, int topk, int window);
csa_status_t csa_sparse_attend(const void *q, const void *kc, const void *vc,
                               const int32_t *idx, int topk,
                               const void *kw, const void *vw, const int32_t *raw_pos0, int R,
                               const int32_t *pos0, int max_pos, int window,
                               const float *sink, float softmax_scale,
                               int B, int Tq, int H, int d, int Nc_cap, csa_dtype_t dt,
                               void *out, float *lse_out,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * hca_attend — HCA dense attention over every completed m'-block.
 * hyper.ai "Method", HCA paragraph (dense attention over heavily compressed
 * entries, no sparse selection, plus a sliding-window branch).
 *
 *   q, out    [B, Tq, H, d]; kc, vc [B, Nc_cap, d] (dt)
 *   the query at t sees entries j < min(floor((t+1)/m_prime), Nc_cap) and,
 *   when window > 0, raw positions max(0,t-W+1)..t from kw/vw as above.
 *   Other arguments as for csa_sparse_attend.
 */
size_t hca_attend_workspace(int B, int Tq, int H, int d, int Nc_cap, int m_prime, int window);
csa_status_t hca_attend(const void *q, const void *kc, const void *vc, int m_prime, int Nc_cap,
                        const void *kw, const void *vw, const int32_t *raw_pos0, int R,
                        int window, const int32_t *pos0, int max_pos,
                        const float *sink, float softmax_scale,
                        int B, int Tq, int H, int d, csa_dtype_t dt,
                        void *out, float *lse_out,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_sparse_attend_kv8 / hca_attend_kv8 — the same attention over caches
 * stored in mixed precision.  hyper.ai "Method", efficiency paragraph: the
 * KV cache keeps its RoPE dimensions in BF16 and the other dimensions in
 * FP8.  Layout read here (the page fixes neither the split nor the scales):
 *   k8     [B, Nc_cap, d/2]  uint8  E4M3 codes of key dims 0 .. d/2-1
 *   krope  [B, Nc_cap, d/2]  bf16   key dims d/2 .. d-1 (the RoPE part)
 *   kscale [B, Nc_cap]       fp32   one scale per key row (codes * scale)
 *   v8     [B, Nc_cap, d]    uint8  E4M3 codes of all value dims (values
 *                                   carry no position encoding)
 *   vscale [B, Nc_cap]       fp32   one scale per value row
 * v8 = vscale = NULL selects the shared-entry variant: each value row is its
 * key row (codes for dims < d/2, the bf16 RoPE half above).
 * Codes are widened exactly to bf16 while the tile is staged in LDS (every
 * E4M3 value is a bf16 value); the key row scale multiplies the fp32 partial
 * logits of the code dims, and the value row scale the fp32 probabilities
 * before they are rounded to bf16 for the product with the values (as on
 * bf16 caches).  With power-of-two scales the results are bitwise those of
 * the bf16 kernels on caches holding code x scale.  q, out, kw, vw are bf16;
 * d = 128.  Other arguments, workspace sizes and errors as csa_sparse_attend
 * and hca_attend.
 */
csa_status_t csa_sparse_attend_kv8(const void *q, const void *k8, const void *krope,
                                   const float *kscale, const void *v8, const float *vscale,
                                   const int32_t *idx, int topk,
                                   const void *kw, const void *vw, const int32_t *raw_pos0, int R,
                                   const int32_t *pos0, int max_pos, int window,
                                   const float *sink, float softmax_scale,
                                   int B, int Tq, int H, int d, int Nc_cap,
                                   void *out, float *lse_out,
                                   void *workspace, size_t workspace_bytes, void *stream);
csa_status_t hca_attend_kv8(const void *q, const void *k8, const void *krope, const float *kscale,
                            const void *v8, const float *vscale, int m_prime, int Nc_cap,
                            const void *kw, const void *vw, const int32_t *raw_pos0, int R,
                            int window, const int32_t *pos0, int max_pos,
                            const float *sink, float softmax_scale,
                            int B, int Tq, int H, int d,
                            void *out, float *lse_out,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_hybrid_attend — the CSA attention and the HCA attention of one hybrid
 * layer pair (hyper.ai "Method": a CSA layer and an HCA layer side by side,
 * each with its sliding-window branch) in one call.
 *
 *   The first 24 arguments are those of csa_sparse_attend and the next 23
 *   those of hca_attend (each prefixed h), with the same meaning, layout and
 *   validation; each problem has its own workspace, sized by its own query
 *   (csa_sparse_attend_workspace / hca_attend_workspace), and the two must not
 *   overlap; out and hout must be different buffers.
 *   Results are bit-identical to the two separate calls.  When both problems
 *   are split decode (Tq = 1) with the same dtype, head dim and query-head
 *   tile shape, one kernel runs the workgroups of both (each with the split
 *   it has in its own call) and one kernel merges the split partials of both;
 *   otherwise the two calls run one after the other on `stream`.  An error in
 *   either part launches nothing; the error text names the part.
 */
csa_status_t csa_hybrid_attend(
    const void *q, const void *kc, const void *vc, const int32_t *idx, int topk,
    const void *kw, const void *vw, const int32_t *raw_pos0, int R,
    const int32_t *pos0, int max_pos, int window, const float *sink, float softmax_scale,
    int B, int Tq, int H, int d, int Nc_cap, csa_dtype_t dt, void *out, float *lse_out,
    void *workspace, size_t workspace_bytes,
    const void *hq, const void *hkc, const void *hvc, int m_prime, int hNc_cap,
    const void *hkw, const void *hvw, const int32_t *hraw_pos0, int hR, int hwindow,
    const int32_t *hpos0, int hmax_pos, const float *hsink, float hsoftmax_scale,
    int hB, int hTq, int hH, int hd, csa_dtype_t hdt, void *hout, float *hlse_out,
    void *hworkspace, size_t hworkspace_bytes, void *stream);

/*
 * csa_hybrid_decode_step — one decode step of a hybrid CSA + HCA layer pair
 * in a single call: the CSA lightning indexer and its top-k selection, the
 * CSA core attention over the selected entries plus the window and sink, and
 * the HCA dense attention (hyper.ai "Method": CSA compresses, scores with a
 * lightning indexer, keeps the top-k and attends with a sliding-window branch;
 * HCA attends densely over its heavily compressed entries; aiboss88 "Technical
 * Principles", CSA bullet: sliding window plus attention sink).  Each of the B
 * sequences has one query token at position pos0[b].
 *
 * The step is described by the struct below; every field has the meaning,
 * layout and validation of the same argument of csa_indexer_topk (the first
 * block), csa_sparse_attend (the second) and hca_attend (the third, fields
 * prefixed h), with Tq = 1 and B, pos0, max_pos, H, d, dt shared by both
 * layers.  idx_out receives the CSA index lists; lse_out / hlse_out may be
 * NULL.  The workspace (size from csa_hybrid_decode_step_workspace) holds the
 * three calls' workspaces behind a block of control words that must be zero
 * before the workspace's first use (allocate it zeroed); every call leaves
 * them zero again, so a workspace is reused as is.  Nothing else may write
 * the workspace between steps.
 *
 * Results are bitwise those of csa_indexer_topk, csa_sparse_attend and
 * hca_attend called one after the other.  The work is enqueued on `stream`
 * as the indexer's kernels (score kernel, row pick), then the CSA and HCA
 * attention as in csa_hybrid_attend (one launch for both problems and one
 * merge of their split partials).  With flags = CSA_STEP_FUSED_TAIL, decode
 * rows on the chunked indexer path (Nc_cap > 12288) with bf16 attention of
 * head dim 128, 33-64 query heads and B <= 1580 instead run both attention
 * problems and both merges in one kernel that orders them through counters
 * in the control words (same results; measured slower on MI355X, where the
 * device-scope counter updates serialise).  The waits inside that kernel are
 * bounded (0.5 s); a wait that runs out (a workspace whose control words were
 * not zero) is counted by the "step_timeout" event counter and leaves the
 * step's outputs undefined.  An invalid field launches nothing; the error
 * text names the part.
 */
#define CSA_STEP_FUSED_TAIL 1u

typedef struct csa_decode_step {
  /* sequences (both layers) */
  int B;
  const int32_t *pos0;        /* [B] device: position of each sequence's query */
  int max_pos;                /* host upper bound of pos0[b] */
  int H, d;                   /* query heads (one KV head), head dim */
  csa_dtype_t dt;             /* attention dtype (CSA_F32 / CSA_BF16) */
  /* CSA lightning indexer + top-k */
  const void *qi, *qi_scale;  /* [B, 1, HI, dI] (FP4 [.., dI/2]); scales as csa_indexer_topk */
  const float *w;             /* [B, 1, HI] */
  const void *kic, *kic_scale;
  int HI, dI, m, topk;
  csa_dtype_t qk_dt;
  int32_t *idx_out;           /* [B, 1, topk] */
  /* CSA core attention */
  const void *q;              /* [B, 1, H, d] */
  const void *kc, *vc;        /* [B, Nc_cap, d] */
  int Nc_cap;                 /* rows per sequence of kc, vc and kic */
  const void *kw, *vw;        /* [B, R, d] raw window rows, or NULL when window == 0 */
  const int32_t *raw_pos0;
  int R, window;
  const float *sink;          /* [H] or NULL */
  float softmax_scale;
  void *out;                  /* [B, 1, H, d] */
  float *lse_out;             /* [B, 1, H] or NULL */
  /* HCA dense attention */
  const void *hq;             /* [B, 1, H, d] */
  const void *hkc, *hvc;      /* [B, hNc_cap, d] */
  int m_prime, hNc_cap;
  const void *hkw, *hvw;      /* [B, hR, d], or NULL when hwindow == 0 */
  const int32_t *hraw_pos0;
  int hR, hwindow;
  const float *hsink;
  float hsoftmax_scale;
  void *hout;                 /* [B, 1, H, d] */
  float *hlse_out;
  unsigned flags;             /* 0, or CSA_STEP_FUSED_TAIL */
} csa_decode_step_t;

size_t csa_hybrid_decode_step_workspace(const csa_decode_step_t *step);
csa_status_t csa_hybrid_decode_step(const csa_decode_step_t *step, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * csa_hybrid_decode_step_static — csa_hybrid_decode_step without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that forbid allocation).  The scratch is a
 * static array of CSA_STEP_SCRATCH_BYTES in device memory, one per device,
 * held until the process ends; the call allocates nothing.  Every call on a
 * device shares that device's array, so calls that overlap on one device
 * (several host threads or streams) race and must be serialised by the
 * caller.  A step whose csa_hybrid_decode_step_workspace exceeds the array
 * returns CSA_WORKSPACE_TOO_SMALL and launches nothing.  The array starts
 * zeroed and every step leaves its control words zero.  Results, arguments
 * and other errors as csa_hybrid_decode_step.
 */
#define CSA_STEP_SCRATCH_BYTES (64u << 20)
csa_status_t csa_hybrid_decode_step_static(const csa_decode_step_t *step, void *stream);

/*
 * csa_grouped_out_proj — grouped output projection after the core attention.
 * hyper.ai "Method", CSA paragraph (the core attention is followed by a
 * grouped output projection that keeps its cost down).  Form implemented:
 * the H heads form G consecutive groups of H/G heads; group j's head outputs
 * of a token, concatenated (K = (H/G) d values), are multiplied by the
 * group's own matrix (stored one row per output, as a linear layer's weight):
 *   y[t, j*dg + n] = sum_k o[t, j*K + k] * w[j, n, k]
 *
 *   o  [T, H, d]   attention outputs (dt), rows of H*d values per token
 *   w  [G, dg, K]  per-group weights (dt), row-major
 *   y  [T, G*dg]   output (dt)
 *   dt ∈ {F32, BF16}; G divides H; K a multiple of 64; dg a multiple of 128;
 *   T * H * d elements under 2 GiB.  Products accumulate in fp32 on the MFMA
 *   units; bf16 outputs are rounded to nearest even.  No workspace.
 */
csa_status_t csa_grouped_out_proj(const void *o, const void *w, int T, int H, int d, int G, int dg,
                                  csa_dtype_t dt, void *y, void *stream);

/*
 * Launch timing, for measurement tools (not part of any computation).
 * While enabled, every kernel launch made by the library is bracketed by a
 * pair of hipEvents recorded on that launch's stream.  csa_profile_query
 * waits for the recorded events of `kernel` and returns (0) the number of
 * launches and their summed GPU duration in milliseconds, or 1 if none were
 * recorded, -1 on a HIP error.  Kernel names: "compress", "indexer_score"
 * (decode scores and per-chunk cut), "indexer_topk" (row select),
 * "indexer_fused" (prefill scores and select in one kernel), "attend_csa",
 * "attend_hca", "attend_pair" (both of csa_hybrid_attend in one kernel),
 * "attend_combine", "decode_tail" (the fused tail of csa_hybrid_decode_step:
 * picks, both attention problems and their merges), "out_proj".
 * csa_profile_reset forgets all records (events are kept for reuse).
 */
void csa_profile_enable(int on);
void csa_profile_reset(void);
int csa_profile_query(const char *kernel, int *count, double *total_ms);

/* Event counters of the current device, for measurement tools: the number of
 * query rows whose top-k selection took the exact fallback path since the
 * last reset ("indexer_prefill_fallback": prefill rows whose candidate set
 * could not settle the top-k; "indexer_decode_fallback": long decode rows whose
 * chunk candidates could not), and "step_timeout": waits of the fused decode
 * step that ran out of time.  Writes the count to *value and, if reset is
 * non-zero, zeroes the counter.  Synchronous (waits for the device); returns 0,
 * 1 for an unknown name or a NULL value, -1 on a HIP error. */
int csa_profile_counter(const char *name, unsigned long long *value, int reset);

#ifdef __cplusplus
}
#endif
#endif /* CSA_MI355X_H */
