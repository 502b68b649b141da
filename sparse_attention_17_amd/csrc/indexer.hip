// Lightning indexer scores + top-k selection.
// Method: DeepSeek-V4 summary (hyper.ai), "Method", CSA paragraph — a
// lightning indexer selects the top-k compressed entries; aiboss88 "Technical
// Principles", CSA bullet (index scores, top-k sparse selection) and FP4 bullet
// (FP4 indexer QK path, FP8 for the extra dynamic range).  Form implemented:
//   I[t,j] = sum_h w[t,h] * max(0, qI[t,h] . KIc_j),   j < floor((t+1)/m)
// then the k largest I[t,.] with equal scores going to the lower j, emitted
// ascending by j and padded with -1.
//
// Scores (MFMA 16x16x32: bf16, fp32 as 8 x 16x16x4; FP8 E4M3 codes, and FP4
// codes times their E8M0 block scale, are widened exactly to bf16 first — the
// native FP8 MFMA accumulates with a few 1e-5 relative error, which would put
// FP8 rows outside a 1e-6 tie band, while bf16 products accumulate in fp32):
//   * prefill tile kernel: (token, head) rows of qI form the A operand (16
//     rows = 16/HI tokens) and 16 entries form B, so each lane receives the HI
//     head dots of one token for one entry and applies ReLU + head weights
//     in-lane;
//   * decode row kernel: one query row; its HI head rows are placed at a
//     different row block for each of 16/HI entry tiles accumulated into one
//     16x16 tile, so all 64 lanes finish one score per 64 entries (HI=4).  It
//     also builds a 12-bit radix histogram of the row's score keys.
// Scores are >= 0 (+0 for ReLU'd zeros), so their fp32 bit patterns order like
// the values.
//
// Top-k:
//   * rows that fit in LDS: one workgroup per row runs an 11/11/10-bit radix
//     select for the k-th largest key tau and the count of ties needed, then an
//     index-ordered compaction keeps keys > tau and the lowest-indexed keys
//     == tau, which is already ascending;
//   * long rows (decode over 32K-262K entries): the histogram gives the bin of
//     tau; a many-workgroup pass writes every index whose key lies above that
//     bin straight to the selection and collects the bin's (key, index) pairs;
//     one workgroup per row then resolves the bin exactly in LDS (radix on the
//     low 20 bits, lowest index among ties) and sorts the k indices.  A row
//     whose boundary bin overflows the candidate buffer falls back to the
//     exact single-workgroup select over the stored scores.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

// Event counters for measurement tools (csa_profile_counter): rows whose
// top-k took the exact fallback select.  Incremented by one lane per event.
__device__ unsigned long long g_counters[CNT_COUNT];

__device__ __forceinline__ void count_event(int which) {
  atomicAdd(&g_counters[which], 1ull);
}

static constexpr int SCORE_WG_ENTRIES = 256;   // prefill tile kernel: 4 waves x 4 tiles x 16
// decode score kernels: entries per chunk (one chunk per workgroup; 1024
// gives two rounds of resident workgroups on a 1M-entry batch, so one round's
// chunk cuts overlap the other's loads)
static constexpr int SCORE_CHUNK = 1024;
static constexpr int SCORE_CPW = 1;            // chunks per score_row_kernel workgroup
static constexpr int SCORE_DEPTH = 3;          // entry groups in flight per wave
static constexpr int H1_BITS = 12;             // first radix digit (key bits 20..31)
static constexpr int H1_BINS = 1 << H1_BITS;
static constexpr int TOPK_NT = 512;
static constexpr int TOPK_LDS_KEYS = 12288;

__host__ __device__ __forceinline__ int nc_pad(int Nc_cap) { return (Nc_cap + 63) & ~63; }

// ---------------- operand loaders: 8 k-values -> one fragment --------------
template <int QK> struct QkTraits;
template <> struct QkTraits<QK_F32> { using F = Frag<float>; };
template <> struct QkTraits<QK_BF16> { using F = Frag<bf16>; };
template <> struct QkTraits<QK_FP8> { using F = Frag<bf16>; };
template <> struct QkTraits<QK_FP4> { using F = Frag<bf16>; };

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two E4M3 codes (bytes 0-1, or 2-3 if HIGH_HALF) -> two packed bf16.  Every E4M3
// value is a bf16 value, so the widening is exact.
template <bool HIGH_HALF>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16(uint32_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, HIGH_HALF));
}

// E2M1 code (low 4 bits) -> fp32 value.
__device__ __forceinline__ float e2m1_val(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, f = c & 1u;
  float mag = e ? (1.f + 0.5f * (float)f) * (float)(1u << e) * 0.5f : 0.5f * (float)f;
  return (c & 8u) ? -mag : mag;
}
// E8M0 code -> 2^(E-127) (E = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_val(uint32_t e) {
  return e ? __uint_as_float(e << 23) : __uint_as_float(0x00400000u);
}

// Fragment of elements k0 .. k0+7 of a row.  FP4: `row` points at packed codes
// and `sc` at the row's E8M0 scales; the FP8 per-row scale is applied later.
// The score kernels give lane group g (lanes 16g..16g+15) the elements
// 8*(g*KC + c) .. +7 for k-chunk c, so a lane's operand bytes are contiguous;
// the MFMA reduction is over all k, so any such relabelling shared by both
// operands gives the same dot product.
template <int QK>
__device__ __forceinline__ void load_qk_frag(typename QkTraits<QK>::F& f, const void* row,
                                             const uint8_t* sc, int k0) {
  if constexpr (QK == QK_F32) {
    frag_load(f, reinterpret_cast<const float*>(row) + k0);
  } else if constexpr (QK == QK_BF16) {
    frag_load(f, reinterpret_cast<const bf16*>(row) + k0);
  } else if constexpr (QK == QK_FP8) {
    const uint2 c = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(row) + k0);
    f.v = u32x4{e4m3x2_to_bf16<false>(c.x), e4m3x2_to_bf16<true>(c.x),
                e4m3x2_to_bf16<false>(c.y), e4m3x2_to_bf16<true>(c.y)};
  } else {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(row) + k0 / 2);
    const float scl = e8m0_val(sc[k0 / 32]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t byte = (c >> (8 * i)) & 0xFF;
      const uint32_t lo = __float_as_uint(e2m1_val(byte & 0xF) * scl) >> 16;
      const uint32_t hi = __float_as_uint(e2m1_val(byte >> 4) * scl) >> 16;
      f.v[i] = lo | (hi << 16);
    }
  }
}

// Split form of load_qk_frag: `load_raw` only issues the loads (so several
// groups can be in flight), `widen` builds the fragment when it is needed.
template <int QK> struct RawFrag { typename QkTraits<QK>::F f; };
template <> struct RawFrag<QK_FP8> { uint2 c; };
template <> struct RawFrag<QK_FP4> { uint32_t c; uint32_t s; };
template <int QK>
__device__ __forceinline__ void load_raw(RawFrag<QK>& r, const void* row, const uint8_t* sc, int k0) {
  if constexpr (QK == QK_FP8) {
    r.c = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(row) + k0);
  } else if constexpr (QK == QK_FP4) {
    r.c = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(row) + k0 / 2);
    r.s = sc[k0 / 32];
  } else {
    load_qk_frag<QK>(r.f, row, sc, k0);
  }
}
template <int QK>
__device__ __forceinline__ typename QkTraits<QK>::F widen(const RawFrag<QK>& r) {
  if constexpr (QK == QK_FP8) {
    typename QkTraits<QK>::F f;
    f.v = u32x4{e4m3x2_to_bf16<false>(r.c.x), e4m3x2_to_bf16<true>(r.c.x),
                e4m3x2_to_bf16<false>(r.c.y), e4m3x2_to_bf16<true>(r.c.y)};
    return f;
  } else if constexpr (QK == QK_FP4) {
    typename QkTraits<QK>::F f;
    const float scl = e8m0_val(r.s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t byte = (r.c >> (8 * i)) & 0xFF;
      const uint32_t lo = __float_as_uint(e2m1_val(byte & 0xF) * scl) >> 16;
      const uint32_t hi = __float_as_uint(e2m1_val(byte >> 4) * scl) >> 16;
      f.v[i] = lo | (hi << 16);
    }
    return f;
  } else {
    return r.f;
  }
}

template <int QK> __host__ __device__ __forceinline__ size_t qk_row_bytes(int dI) {
  if constexpr (QK == QK_F32) return (size_t)dI * 4;
  else if constexpr (QK == QK_BF16) return (size_t)dI * 2;
  else if constexpr (QK == QK_FP8) return (size_t)dI;
  else return (size_t)dI / 2;
}

__device__ __forceinline__ int row_len(const IndexerArgs& a, int b, int t) {
  return max(0, min((a.pos0[b] + t + 1) / a.m, a.Nc_cap));
}

// Workspace carve-up for the long-row path (per query row; nch = score chunks):
//   scores [rows][ldo] f32 | meta [rows][nch][2] u32 (kept count, cut) |
//   cand [rows][nch * SCORE_CHUNK][2] u32 (key, entry), chunk c's kept entries
//   at slots c * cap ..  (cap = the row's per-chunk capacity)
// Every score workgroup owns one chunk's slots, so no atomics are needed.
struct LongWs {
  float* scores;
  uint32_t *meta, *cand;
  int nch;
};
__host__ __device__ __forceinline__ int row_chunks(int Nc_cap) { return (Nc_cap + SCORE_CHUNK - 1) / SCORE_CHUNK; }
__host__ __device__ __forceinline__ LongWs long_ws(void* ws, int rows, int Nc_cap) {
  LongWs w;
  w.nch = row_chunks(Nc_cap);
  char* p = reinterpret_cast<char*>(ws);
  w.scores = reinterpret_cast<float*>(p);
  p += (size_t)rows * nc_pad(Nc_cap) * 4;
  w.meta = reinterpret_cast<uint32_t*>(p);
  p += (size_t)rows * ((w.nch * 2 + 3) & ~3) * 4;
  w.cand = reinterpret_cast<uint32_t*>(p);
  return w;
}
static size_t long_ws_bytes(int rows, int Nc_cap) {
  const int nch = row_chunks(Nc_cap);
  return (size_t)rows * ((size_t)nc_pad(Nc_cap) * 4 + (size_t)((nch * 2 + 3) & ~3) * 4 +
                         (size_t)nch * SCORE_CHUNK * 8);
}
// Candidate slots per chunk for the row select: a power of two in
// [32, SCORE_CHUNK] near four times the chunk's expected share of the top k;
// the chunk keeps its kc = 3/4 of that (three times its share) largest keys
// plus whatever shares the kc-th key's 20-bit prefix, up to the slots.
__host__ __device__ __forceinline__ int chunk_cap_n(int k, int n) {
  const long long want = (4LL * k * SCORE_CHUNK + n - 1) / n;
  int cap = 32;
  while (cap < want && cap < SCORE_CHUNK) cap <<= 1;
  return cap;
}
__host__ __device__ __forceinline__ int chunk_keep(int k, int n) {
  const int cap = chunk_cap_n(k, n);
  return cap < SCORE_CHUNK ? cap - cap / 4 : SCORE_CHUNK;
}
static constexpr uint32_t CUT_ALL = 0xFFFFFFFFu;   // the chunk kept every entry
static bool use_long_path(int Tq, int Nc_cap) { return Tq <= 4 && Nc_cap > TOPK_LDS_KEYS; }

// Scanning bins from the top down, find the bin where the running count first
// reaches `need`; out[0] = bin, out[1] = count strictly above it.
template <int NT>
__device__ void find_bin(const uint32_t* hist, int nbins, uint32_t need, uint32_t* scan,
                         uint32_t* out) {
  const int per = nbins / NT;
  const int tid = threadIdx.x;
  const int hi = nbins - tid * per;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[hi - 1 - i];
  uint32_t tot;
  const uint32_t excl = block_excl_scan<NT>(local, scan, &tot);
  if (excl < need && excl + local >= need) {
    uint32_t cum = excl;
    for (int i = 0; i < per; ++i) {
      const uint32_t h = hist[hi - 1 - i];
      if (cum + h >= need) { out[0] = hi - 1 - i; out[1] = cum; break; }
      cum += h;
    }
  }
  __syncthreads();
}

// Top-down search within a wave: given cnt(i) for bins [0, nb) (nb = 64*per),
// the bin where the running count from the top first reaches `need`, and the
// count strictly above it (all lanes get the result).
template <typename Cnt>
__device__ __forceinline__ void wave_top_bin(int per, uint32_t need, Cnt cnt, uint32_t& bin,
                                             uint32_t& above) {
  const int lane = threadIdx.x & 63;
  const int hi = 64 * per - lane * per;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += cnt(hi - 1 - i);
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t excl = incl - local;
  const bool mine = excl < need && incl >= need;
  uint32_t bb = 0, ab = 0;
  if (mine) {
    uint32_t cum = excl;
    for (int i = 0; i < per; ++i) {
      const uint32_t h = cnt(hi - 1 - i);
      if (cum + h >= need) { bb = hi - 1 - i; ab = cum; break; }
      cum += h;
    }
  }
  const uint64_t m = __ballot(mine);
  const int src = m ? __ffsll((unsigned long long)m) - 1 : 0;
  bin = (uint32_t)__builtin_amdgcn_readlane((int)bb, src);
  above = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
}

// End of a decode score workgroup (256 threads): keep the chunk's entries at
// or above its cut, in index order, in the chunk's candidate slots.  The cut
// is the 20-bit key prefix (key >> 12) of the chunk's kc-th largest key: its
// 12-bit digit comes from the digit histogram (every thread first sums 16
// bins, then each wave scans those sums), the next 8 bits from a histogram of
// the entries inside that digit.  Every wave finds the cut by itself, so the
// whole step needs three barriers.  sk holds the chunk's nloc keys, hist
// their 12-bit digit histogram; cw is 256 + 256 + 4 words of scratch.
__device__ void chunk_cut(const IndexerArgs& a, const LongWs& L, int row, int chunk, int n, int c0,
                          int nloc, const uint32_t* sk, const uint32_t* hist, uint32_t* cw) {
  constexpr int PER = SCORE_CHUNK / 256;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kc = chunk_keep(a.topk, n), cap = chunk_cap_n(a.topk, n);
  const int i0 = tid * PER;
  uint32_t* part = cw;                                       // 256 sums of 16 digit bins
  uint32_t* h8 = cw + 256;                                   // second-level histogram
  uint32_t* wtot = cw + 512;                                 // per-wave counts
  uint32_t cut = 0;
  const bool dropped = nloc > kc;                            // uniform
  if (dropped) {
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += hist[16 * tid + i];
    part[tid] = sum;
    h8[tid] = 0;
    __syncthreads();
    uint32_t grp, above;
    wave_top_bin(4, (uint32_t)kc, [&](int i) { return part[i]; }, grp, above);
    uint32_t d1, above1;
    wave_top_bin(1, (uint32_t)kc - above, [&](int i) { return i < 16 ? hist[16 * grp + i] : 0u; }, d1, above1);
    d1 += 16 * grp;
    above += above1;
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (i0 + q < nloc && (sk[i0 + q] >> 20) == d1) atomicAdd(&h8[(sk[i0 + q] >> 12) & 255u], 1u);
    __syncthreads();
    uint32_t d2, above2;
    wave_top_bin(4, (uint32_t)kc - above, [&](int i) { return h8[i]; }, d2, above2);
    cut = (d1 << 8) | d2;
  }
  uint32_t keep = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (i0 + q < nloc && (sk[i0 + q] >> 12) >= cut) keep |= 1u << q;
  const uint32_t cnt = (uint32_t)__popc(keep);
  const uint32_t incl = wave_incl_scan(cnt);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  uint32_t pos = incl - cnt, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = wtot[w];
    pos += w < wave ? v : 0u;
    tot += v;
  }
  uint2* cd = reinterpret_cast<uint2*>(L.cand) + (size_t)row * L.nch * SCORE_CHUNK + (size_t)chunk * cap;
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if ((keep >> q) & 1u) {
      if (pos < (uint32_t)cap) cd[pos] = uint2{sk[i0 + q], (uint32_t)(c0 + i0 + q)};
      ++pos;
    }
  if (tid == 0) {
    L.meta[((size_t)row * L.nch + chunk) * 2] = tot;
    L.meta[((size_t)row * L.nch + chunk) * 2 + 1] = dropped ? cut : CUT_ALL;
  }
}

// --------------------------- prefill score tile ----------------------------
template <int QK, int DI, int HI>
__global__ __launch_bounds__(256) void score_tile_kernel(IndexerArgs a) {
  constexpr int TT = 16 / HI;        // tokens per workgroup
  constexpr int KC = DI / 32;        // 32-wide k chunks
  using F = typename QkTraits<QK>::F;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * TT;
  const int e_wg = blockIdx.x * SCORE_WG_ENTRIES;
  const int t_last = min(t0 + TT, a.Tq) - 1;
  const int ne_max = row_len(a, b, t_last);
  if (e_wg >= ne_max) return;

  const int r = lane & 15, g = lane >> 4;
  const int tq = t0 + r / HI, hq = r % HI;
  F qa[KC];
  const uint8_t* qsc = nullptr;
  const size_t qrow = ((size_t)b * a.Tq + tq) * HI + hq;
  const char* qptr = reinterpret_cast<const char*>(a.qi) + qrow * qk_row_bytes<QK>(DI);
  if constexpr (QK == QK_FP4) qsc = reinterpret_cast<const uint8_t*>(a.qi_scale) + qrow * (DI / 32);
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (tq < a.Tq) load_qk_frag<QK>(qa[c], qptr, qsc, 8 * (g * KC + c));
    else frag_zero(qa[c]);
  }
  float wr[4];
  int trow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 4 * g + i;
    const int t = t0 + rr / HI, h = rr % HI;
    trow[i] = t;
    float wv = 0.f;
    if (t < a.Tq) {
      const size_t wi = ((size_t)b * a.Tq + t) * HI + h;
      wv = a.w[wi];
      if constexpr (QK == QK_FP8) wv *= reinterpret_cast<const float*>(a.qi_scale)[wi];
    }
    wr[i] = wv;
  }
  const int ldo = nc_pad(a.Nc_cap);
  float* ws = reinterpret_cast<float*>(a.ws);

#pragma unroll 1
  for (int tile = 0; tile < 4; ++tile) {
    const int e0 = e_wg + (wave * 4 + tile) * 16;
    if (e0 >= ne_max) break;
    const int e = e0 + r;
    const bool ev = e < ne_max;
    const size_t krow = (size_t)b * a.Nc_cap + (ev ? e : 0);
    const char* kptr = reinterpret_cast<const char*>(a.kic) + krow * qk_row_bytes<QK>(DI);
    const uint8_t* ksc = nullptr;
    if constexpr (QK == QK_FP4) ksc = reinterpret_cast<const uint8_t*>(a.kic_scale) + krow * (DI / 32);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      F kb;
      load_qk_frag<QK>(kb, kptr, ksc, 8 * (g * KC + c));
      mma16(acc, qa[c], kb);
    }
    float cs = 1.f;
    if constexpr (QK == QK_FP8) cs = reinterpret_cast<const float*>(a.kic_scale)[krow];
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = acc[i];
      s[i / HI] = fmaf(wr[i], x > 0.f ? x : 0.f, s[i / HI]);
    }
#pragma unroll
    for (int u = 0; u < 4 / HI; ++u) {
      const int t = trow[u * HI];
      if (t < a.Tq && ev) {
        if (e < row_len(a, b, t)) ws[((size_t)b * a.Tq + t) * ldo + e] = s[u] * cs + 0.f;
      }
    }
  }
}

// ---------------------------- decode score row -----------------------------
template <int QK, int DI, int HI>
__global__ __launch_bounds__(256) void score_row_kernel(IndexerArgs a) {
  constexpr int KC = DI / 32;
  constexpr int TPC = 16 / HI;        // 16-entry tiles accumulated into one 16x16 tile
  constexpr int EPC = 16 * TPC;       // entries per accumulator (64 for HI=4)
  constexpr int SPL = 4 / HI;         // scores per lane per accumulator
  using F = typename QkTraits<QK>::F;
  __shared__ uint32_t hist[H1_BINS];
  __shared__ uint32_t sk[SCORE_CHUNK];
  __shared__ uint32_t cut_ws[516];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowJ rj = xcd_rows(blockIdx.x, a.B * a.Tq, gridDim.x / (a.B * a.Tq));
  const int row = rj.row;
  const int b = row / a.Tq, t = row % a.Tq;
  const int n = row_len(a, b, t);
  const int chunk0 = rj.j * SCORE_CPW;
  if (chunk0 * SCORE_CHUNK >= n) return;
  LongWs L = long_ws(a.ws, a.B * a.Tq, a.Nc_cap);

  const int r = lane & 15, g = lane >> 4;
  const size_t rb = qk_row_bytes<QK>(DI);
  const char* kbase = reinterpret_cast<const char*>(a.kic) + (size_t)b * a.Nc_cap * rb;
  const uint8_t* sbase = nullptr;
  if constexpr (QK == QK_FP4) sbase = reinterpret_cast<const uint8_t*>(a.kic_scale) + (size_t)b * a.Nc_cap * (DI / 32);
  const float* fsc = nullptr;
  if constexpr (QK == QK_FP8) fsc = reinterpret_cast<const float*>(a.kic_scale) + (size_t)b * a.Nc_cap;
  float* srow = L.scores + (size_t)row * nc_pad(a.Nc_cap);

  // one group = EPC entries of the chunk ending at c1: the B fragments plus
  // (FP8) the per-entry scales of the entries this lane will score
  using R = RawFrag<QK>;
  auto load_group = [&](int e0, int c1, R (&kb)[TPC][KC], float (&ks)[SPL]) {
#pragma unroll
    for (int u = 0; u < TPC; ++u) {
      const int e = min(e0 + 16 * u + r, c1 - 1);
#pragma unroll
      for (int c = 0; c < KC; ++c)
        load_raw<QK>(kb[u][c], kbase + (size_t)e * rb,
                     QK == QK_FP4 ? sbase + (size_t)e * (DI / 32) : nullptr, 8 * (g * KC + c));
    }
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      if constexpr (QK == QK_FP8) ks[s] = fsc[min(e0 + 16 * ((4 * g) / HI + s) + r, c1 - 1)];
      else ks[s] = 1.f;
    }
  };

  // DEPTH groups in flight per wave; a chunk's groups are fully unrolled and
  // branch-free (loads clamp to the chunk, stores are masked).  The first
  // chunk's groups are requested before the query and the head weights, so
  // the two latencies overlap.  A workgroup scores SCORE_CPW consecutive
  // chunks and requests the next chunk's first groups before cutting the
  // current one, so the cut overlaps those loads.
  constexpr int STRIDE = 4 * EPC;
  constexpr int NG = (SCORE_CHUNK + STRIDE - 1) / STRIDE;
  constexpr int DEPTH = NG < SCORE_DEPTH ? NG : SCORE_DEPTH;
  R kb[DEPTH][TPC][KC];
  float ks[DEPTH][SPL];
  {
    const int c0 = chunk0 * SCORE_CHUNK, c1 = min(n, c0 + SCORE_CHUNK);
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) load_group(c0 + wave * EPC + j * STRIDE, c1, kb[j], ks[j]);
  }
  // A operands: for tile u the query's HI head rows sit at rows u*HI .. u*HI+HI-1
  const int hq = r % HI, uq = r / HI;
  const size_t qrow = ((size_t)b * a.Tq + t) * HI + hq;
  const char* qptr = reinterpret_cast<const char*>(a.qi) + qrow * qk_row_bytes<QK>(DI);
  const uint8_t* qsc = nullptr;
  if constexpr (QK == QK_FP4) qsc = reinterpret_cast<const uint8_t*>(a.qi_scale) + qrow * (DI / 32);
  // FP8: the codes themselves are the operands of the FP8 MFMA (E4M3 x E4M3
  // products are exact in its fp32 accumulation, as in the bf16 MFMA on the
  // exactly widened codes); the row scales multiply the weights and scores.
  constexpr bool NATIVE8 = QK == QK_FP8;
  F qa[NATIVE8 ? 1 : TPC][KC];
  uint64_t qa8[NATIVE8 ? TPC : 1][KC];
  if constexpr (NATIVE8) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const uint64_t qc = *reinterpret_cast<const uint64_t*>(qptr + 8 * (g * KC + c));
#pragma unroll
      for (int u = 0; u < TPC; ++u) qa8[u][c] = u == uq ? qc : 0ull;
    }
  } else {
    F qv[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) load_qk_frag<QK>(qv[c], qptr, qsc, 8 * (g * KC + c));
#pragma unroll
    for (int u = 0; u < TPC; ++u)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (u == uq) qa[u][c] = qv[c];
        else frag_zero(qa[u][c]);
      }
  }
  // weights of the head rows this lane receives: rows 4g+i -> head (4g+i) % HI
  float wr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t wi = ((size_t)b * a.Tq + t) * HI + ((4 * g + i) % HI);
    float wv = a.w[wi];
    if constexpr (QK == QK_FP8) wv *= reinterpret_cast<const float*>(a.qi_scale)[wi];
    wr[i] = wv;
  }

  // process one group of the chunk [c0, c1): MFMAs, ReLU + head weights, store,
  // chunk key copy and histogram
  auto process = [&](int e0, int c0, int c1, const R (&cur)[TPC][KC], const float (&cscl)[SPL]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < TPC; ++u)
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if constexpr (NATIVE8)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)qa8[u][c], __builtin_bit_cast(long, cur[u][c].c),
                                                          acc, 0, 0, 0);
        else
          mma16(acc, qa[u][c], widen<QK>(cur[u][c]));
      }
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      const int u = (4 * g) / HI + s;
      const int e = e0 + 16 * u + r;
      float sc = 0.f;
#pragma unroll
      for (int h = 0; h < HI; ++h) {
        const float x = acc[s * HI + h];
        sc = fmaf(wr[s * HI + h], x > 0.f ? x : 0.f, sc);
      }
      if (e < c1) {
        if constexpr (QK == QK_FP8) sc *= cscl[s];
        sc += 0.f;
        srow[e] = sc;
        sk[e - c0] = __float_as_uint(sc);
        atomicAdd(&hist[__float_as_uint(sc) >> (32 - H1_BITS)], 1u);
      }
    }
  };

#pragma unroll 1
  for (int ci = 0; ci < SCORE_CPW; ++ci) {
    const int chunk = chunk0 + ci;
    const int c0 = chunk * SCORE_CHUNK;
    if (c0 >= n) break;                                      // uniform
    const int c1 = min(n, c0 + SCORE_CHUNK);
    for (int i = threadIdx.x; i < H1_BINS; i += 256) hist[i] = 0;
    __syncthreads();
    const int ew = c0 + wave * EPC;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      process(ew + j * STRIDE, c0, c1, kb[j % DEPTH], ks[j % DEPTH]);
      if (j + DEPTH < NG) load_group(ew + (j + DEPTH) * STRIDE, c1, kb[j % DEPTH], ks[j % DEPTH]);
    }
    __syncthreads();
    const int n0 = c0 + SCORE_CHUNK;                         // the next chunk
    if (ci + 1 < SCORE_CPW && n0 < n) {
      const int n1 = min(n, n0 + SCORE_CHUNK);
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) load_group(n0 + wave * EPC + j * STRIDE, n1, kb[j], ks[j]);
    }
    if (n > a.topk) chunk_cut(a, L, row, chunk, n, c0, c1 - c0, sk, hist, cut_ws);
    __syncthreads();                                         // hist and sk are reused
  }
}

// ------------------------ decode score row, native FP4 ------------------------
// v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands: lane (c = l%16,
// kb = l/16) supplies 32 FP4 values (16 bytes) of column c / row c for the
// k-block kb and the E8M0 scale of that block.  An entry has DI/32 blocks, so
// one 128-deep k column holds 4/(DI/32) entries; the query's four head rows are
// placed, per entry slot p, at rows 4p..4p+3 and only in the k-blocks of that
// slot, so the accumulator gives lane group g the four head dots of entry
// e0 + 16g + c, exactly as in the generic decode kernel.
template <int DI>
__global__ __launch_bounds__(256) void score_row_fp4_kernel(IndexerArgs a) {
  constexpr int HI = 4;
  constexpr int KBE = DI / 32;                 // k-blocks per entry
  constexpr int EPCOL = 4 / KBE;               // entries per 128-deep column
  constexpr int NM = KBE;                      // MFMAs per 64 entries
  constexpr int EPC = 64;
  constexpr int RB = DI / 2;                   // bytes per packed row
  __shared__ uint32_t hist[H1_BINS];
  __shared__ uint32_t sk[SCORE_CHUNK];
  __shared__ uint32_t cut_ws[516];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowJ rj = xcd_rows(blockIdx.x, a.B * a.Tq, gridDim.x / (a.B * a.Tq));
  const int row = rj.row, chunk = rj.j;
  const int b = row / a.Tq, t = row % a.Tq;
  const int n = row_len(a, b, t);
  const int c0 = chunk * SCORE_CHUNK;
  if (c0 >= n) return;
  const int c1 = min(n, c0 + SCORE_CHUNK);
  LongWs L = long_ws(a.ws, a.B * a.Tq, a.Nc_cap);
  for (int i = threadIdx.x; i < H1_BINS; i += 256) hist[i] = 0;

  const int c = lane & 15, kb = lane >> 4;
  const int half = kb % KBE;
  // A operands: row r = 4p + h holds q_h in the k-blocks of entry slot p
  i32x8 qa[NM];
  int qs[NM];
  {
    const int h = c % 4, p = c / 4;
    const size_t qrow = ((size_t)b * a.Tq + t) * HI + h;
    const u32x4 qv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.qi) + qrow * RB + 16 * half);
    const int qsv = reinterpret_cast<const uint8_t*>(a.qi_scale)[qrow * KBE + half];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const bool on = (m * EPCOL + kb / KBE) == p;
      qa[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (on) { qa[m][0] = qv[0]; qa[m][1] = qv[1]; qa[m][2] = qv[2]; qa[m][3] = qv[3]; }
      qs[m] = on ? qsv : 127;
    }
  }
  float wr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) wr[i] = a.w[((size_t)b * a.Tq + t) * HI + i];
  __syncthreads();

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.kic) + (size_t)b * a.Nc_cap * RB;
  const uint8_t* sbase = reinterpret_cast<const uint8_t*>(a.kic_scale) + (size_t)b * a.Nc_cap * KBE;
  float* srow = L.scores + (size_t)row * nc_pad(a.Nc_cap);

  auto load_group = [&](int e0, u32x4 (&kv)[NM], int (&ks)[NM]) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int e = min(e0 + 16 * (m * EPCOL + kb / KBE) + c, c1 - 1);
      kv[m] = *reinterpret_cast<const u32x4*>(kbase + (size_t)e * RB + 16 * half);
      ks[m] = sbase[(size_t)e * KBE + half];
    }
  };
  auto process = [&](int e0, const u32x4 (&kv)[NM], const int (&ks)[NM]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const i32x8 bv = i32x8{(int)kv[m][0], (int)kv[m][1], (int)kv[m][2], (int)kv[m][3], 0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[m], bv, acc, 4, 4, 0, qs[m], 0, ks[m]);
    }
    const int e = e0 + lane;
    float sc = 0.f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float x = acc[h];
      sc = fmaf(wr[h], x > 0.f ? x : 0.f, sc);
    }
    if (e < c1) {
      sc += 0.f;
      srow[e] = sc;
      sk[e - c0] = __float_as_uint(sc);
      atomicAdd(&hist[__float_as_uint(sc) >> (32 - H1_BITS)], 1u);
    }
  };
  constexpr int STRIDE = 4 * EPC;
  u32x4 kvA[NM], kvB[NM];
  int ksA[NM], ksB[NM];
  int e0 = c0 + wave * EPC;
  if (e0 < c1) load_group(e0, kvA, ksA);
  if (e0 + STRIDE < c1) load_group(e0 + STRIDE, kvB, ksB);
#pragma unroll 1
  for (; e0 < c1; e0 += 2 * STRIDE) {
    process(e0, kvA, ksA);
    if (e0 + 2 * STRIDE < c1) load_group(e0 + 2 * STRIDE, kvA, ksA);
    if (e0 + STRIDE < c1) {
      process(e0 + STRIDE, kvB, ksB);
      if (e0 + 3 * STRIDE < c1) load_group(e0 + 3 * STRIDE, kvB, ksB);
    }
  }
  __syncthreads();
  if (n > a.topk) chunk_cut(a, L, row, chunk, n, c0, c1 - c0, sk, hist, cut_ws);
}

// --------------------------- shared select helpers --------------------------
template <int NT>
struct TopkSmem {
  uint32_t hist[2048];
  uint32_t scan[NT / 64];
  uint32_t res[2];
};

// Exact select of one row whose keys are in `row` (LDS or global), n > k.
template <int NT>
__device__ void select_row(TopkSmem<NT>& sm, const uint32_t* __restrict__ row, int n, int k,
                           int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  if (tid == 0) { sm.res[0] = 0; sm.res[1] = 0; }
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const int sh = p == 0 ? 21 : (p == 1 ? 10 : 0);
    const int nb = p == 2 ? 1024 : 2048;
    for (int i = tid; i < nb; i += NT) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = row[i];
      if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin<NT>(sm.hist, nb, need, sm.scan, sm.res);
    prefix |= sm.res[0] << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    need -= sm.res[1];
    __syncthreads();
  }
  const uint32_t tau = prefix, need_eq = need;
  uint32_t base = 0, eq_seen = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < n; c0 += NT) {
    const int i = c0 + tid;
    const uint32_t key = i < n ? row[i] : 0u;
    const uint32_t is_gt = (i < n && key > tau) ? 1u : 0u;
    const uint32_t is_eq = (i < n && key == tau) ? 1u : 0u;
    uint32_t tot_eq;
    const uint32_t eq_x = block_excl_scan<NT>(is_eq, sm.scan, &tot_eq);
    const uint32_t take = is_gt | ((is_eq && eq_seen + eq_x < need_eq) ? 1u : 0u);
    uint32_t tot_take;
    const uint32_t pos = block_excl_scan<NT>(take, sm.scan, &tot_take);
    if (take && base + pos < (uint32_t)k) {
      idx_out[base + pos] = i;
      if (score_out) score_out[base + pos] = __uint_as_float(key);
    }
    base += tot_take;
    eq_seen += tot_eq;
    if (base >= (uint32_t)k) break;
  }
}

__device__ __forceinline__ void write_all_eligible(int n, int k, const uint32_t* src,
                                                   int32_t* idx, float* sco, int nt) {
  for (int i = threadIdx.x; i < k; i += nt) {
    idx[i] = i < n ? i : -1;
    if (sco) sco[i] = i < n ? __uint_as_float(src[i]) : -INFINITY;
  }
}

// ------------------------- per-row LDS top-k kernel -------------------------
__global__ __launch_bounds__(TOPK_NT) void topk_row_kernel(IndexerArgs a) {
  __shared__ TopkSmem<TOPK_NT> sm;
  __shared__ uint32_t rowbuf[TOPK_LDS_KEYS];
  const int t = blockIdx.x, b = blockIdx.y;
  const int n = row_len(a, b, t);
  const size_t orow = ((size_t)b * a.Tq + t) * a.topk;
  int32_t* idx = a.idx_out + orow;
  float* sco = a.score_out ? a.score_out + orow : nullptr;
  const uint32_t* src =
      reinterpret_cast<const uint32_t*>(a.ws) + ((size_t)b * a.Tq + t) * nc_pad(a.Nc_cap);
  if (n <= a.topk) {
    write_all_eligible(n, a.topk, src, idx, sco, TOPK_NT);
    return;
  }
  if (n <= TOPK_LDS_KEYS) {
    for (int i = threadIdx.x; i < n; i += TOPK_NT) rowbuf[i] = src[i];
    __syncthreads();
    select_row<TOPK_NT>(sm, rowbuf, n, a.topk, idx, sco);
  } else {
    select_row<TOPK_NT>(sm, src, n, a.topk, idx, sco);
  }
}

// ------------------------------ long-row path ------------------------------
// One workgroup per query row picks the row's k largest keys among the
// chunks' candidates.  Candidate slot (chunk c, j) holds the j-th kept entry
// of chunk c; slots in (c, j) order are in ascending entry order, so the
// lowest-index rule among equal keys is slot order and the output needs no
// sort.  The pick is exact when every chunk's dropped entries lie below the
// selected threshold tau (tau >= cut << 12) and no chunk overflowed its slots;
// otherwise the row is selected exactly from the stored scores.
static constexpr int PICK_NT = 1024;
static constexpr int PICK_NW = PICK_NT / 64;
static constexpr int PICK_MAXCH = 4096;        // rows up to 8M entries
static constexpr int PICK_MAXPER = 30;         // candidate slots per thread, largest body
static constexpr int PICK_WORDS = PICK_MAXPER * PICK_NT / 32;
static constexpr int PICK_STASH = 16384;       // slots whose selected entry is kept in LDS
static constexpr int PICK_BINS = 4096;         // 12-bit radix digits

struct PickSmem {
  uint32_t hist[2][PICK_BINS];                 // alternating digit histograms
  uint32_t ccnt[PICK_MAXCH];                   // kept count per chunk (clamped to cap)
  uint32_t ccut[PICK_MAXCH];                   // cut key prefix per chunk
  uint32_t bm_gt[PICK_WORDS];                  // output bitmaps over slots
  uint32_t bm_eq[PICK_WORDS];
  uint32_t sel[PICK_STASH];                    // entry index of selected slots
  uint32_t wv[4][PICK_NW];                     // per-wave partials
  uint32_t res[3];                             // bin, count above it, count in it
};
static_assert(sizeof(TopkSmem<PICK_NT>) <= sizeof(PickSmem), "fallback select aliases PickSmem");

// Sum of the per-wave totals w[0 .. wave-1] (wave = this thread's wave):
// lane i < PICK_NW reads w[i] once and a masked wave sum replaces a serial
// walk over the totals.
__device__ __forceinline__ uint32_t waves_below(const uint32_t* w, int wave) {
  const int lane = threadIdx.x & 63;
  return wave_sum_u32(lane < wave ? w[lane] : 0u);           // wave < PICK_NW <= 64
}

struct PickRow {
  int row, n, k, nch, cap, lg, nslot;
  const uint2* meta;
  const uint2* cand;
  const uint32_t* src;
  int32_t* idx;
  float* sco;
};

// Select for one row whose nslot fits PER slots per thread.  Slot s holds
// (key, entry) of the (s mod cap)-th kept entry of chunk s / cap; thread tid
// holds slots q * PICK_NT + tid (coalesced loads).  Every loop runs exactly
// PER times, and the output bitmaps are built from wave ballots.
template <int PER>
__device__ __forceinline__ void pick_body(PickSmem& sm, const PickRow& R) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr uint2 EMPTY = {0u, 0xFFFFFFFFu};
  const int k = R.k, cap = R.cap, lg = R.lg, nslot = R.nslot, nch = R.nch;

  // ---- 1. candidate slots and chunk records, requested together ----
  uint2 kv[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) kv[q] = R.cand[min(q * PICK_NT + tid, nslot - 1)];
  uint32_t part = 0;
  int bad = 0;
  for (int c = tid; c < nch; c += PICK_NT) {
    const uint2 r = R.meta[c];
    sm.ccnt[c] = min(r.x, (uint32_t)cap);
    sm.ccut[c] = r.y;
    bad |= r.x > (uint32_t)cap;
    part += min(r.x, (uint32_t)cap);
  }
  for (int i = tid; i < PICK_BINS; i += PICK_NT) sm.hist[0][i] = 0;
  __syncthreads();

  // ---- 2. mask empty slots; candidate total, key range, overflow ----
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int s = q * PICK_NT + tid;
    const bool ok = s < nslot && (s & (cap - 1)) < (int)sm.ccnt[min(s >> lg, PICK_MAXCH - 1)];
    kv[q].x = ok ? kv[q].x : EMPTY.x;
    kv[q].y = ok ? kv[q].y : EMPTY.y;
    kmin = ok ? min(kmin, kv[q].x) : kmin;
    kmax = ok ? max(kmax, kv[q].x) : kmax;
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  part = wave_sum_u32(part);
  bad = wave_max_u32((uint32_t)bad) != 0u;
  if (lane == 0) { sm.wv[0][wave] = part; sm.wv[1][wave] = kmin; sm.wv[2][wave] = kmax; sm.wv[3][wave] = bad; }
  __syncthreads();
  uint32_t total = 0;
  kmin = 0xFFFFFFFFu; kmax = 0; bad = 0;
#pragma unroll
  for (int w = 0; w < PICK_NW; ++w) {
    total += sm.wv[0][w];
    kmin = min(kmin, sm.wv[1][w]);
    kmax = max(kmax, sm.wv[2][w]);
    bad |= sm.wv[3][w];
  }
  bad |= total < (uint32_t)k;

  // ---- 3. exact radix select of the k-th largest candidate key ----
  // The candidates are the tops of their chunks and share leading bits, so
  // the 12-bit digits start at the highest bit where the smallest and largest
  // key differ; that spreads them over the bins.
  uint32_t tau = kmin, need = (uint32_t)k;
  if (!bad && kmin != kmax) {
    const int top = 31 - __clz((int)(kmin ^ kmax));
    uint32_t prefix = top >= 31 ? 0u : (kmin & ~((2u << top) - 1u));
    uint32_t pmask = top >= 31 ? 0u : ~((2u << top) - 1u);
    int buf = 0;
#pragma unroll 1
    for (int hi = top; hi >= 0; hi -= 12) {
      const int sh = hi >= 11 ? hi - 11 : 0;
      const int nb = 1 << (hi - sh + 1);
      const int nbs = max(nb, PICK_NT);                       // bins scanned
      uint32_t* hist = sm.hist[buf];
      for (int i = tid; i < PICK_BINS; i += PICK_NT) sm.hist[buf ^ 1][i] = 0;   // next pass's buffer
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const uint2 v = kv[q];
        if (v.y != EMPTY.y && (v.x & pmask) == prefix) atomicAdd(&hist[(v.x >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      // top-down scan: thread tid owns bins [nbs - pb*(tid+1), nbs - pb*tid)
      const int pb = nbs / PICK_NT;
      const int hb = nbs - pb * tid;
      uint32_t local = 0;
      for (int i = 0; i < pb; ++i) local += hist[hb - 1 - i];
      const uint32_t incl = wave_incl_scan(local);
      if (lane == 63) sm.wv[0][wave] = incl;
      __syncthreads();
      uint32_t before = incl - local;
      before += waves_below(sm.wv[0], wave);
      if (before < need && before + local >= need) {
        uint32_t cum = before;
        for (int i = 0; i < pb; ++i) {
          const uint32_t h = hist[hb - 1 - i];
          if (cum + h >= need) {
            sm.res[0] = (uint32_t)(hb - 1 - i); sm.res[1] = cum; sm.res[2] = h;
            break;
          }
          cum += h;
        }
      }
      __syncthreads();
      prefix |= sm.res[0] << sh;
      pmask |= (uint32_t)(nb - 1) << sh;
      need -= sm.res[1];
      buf ^= 1;
      // Every key in the bin is taken: tau = the bin's floor (bits below sh
      // zero) then selects the same set (the keys above it plus the whole bin)
      // and the later passes are skipped.  Only for sh <= 12, where the floor
      // and the k-th key compare alike against the chunk cuts (multiples of
      // 2^12) in the safety check below.
      if (sm.res[2] == need && sh <= 12) break;
    }
    tau = prefix;
  }
  // the chunks' dropped entries must all lie below tau
  int unsafe = bad;
  if (!bad)
    for (int c = tid; c < nch; c += PICK_NT) {
      const uint32_t cut = sm.ccut[c];
      unsafe |= cut != CUT_ALL && tau < (cut << 12);
    }
  // slot bitmaps of keys > tau and keys == tau, one ballot per 64 slots (each
  // word has one writer: no atomics, no clearing); selected entries kept
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const uint2 v = kv[q];
    const int s = q * PICK_NT + tid;
    const bool valid = v.y != EMPTY.y;
    const bool gt = valid && v.x > tau, eq = valid && v.x == tau;
    if ((gt || eq) && s < PICK_STASH) sm.sel[s] = v.y;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      const int w0 = (q * PICK_NT + wave * 64) >> 5;
      sm.bm_gt[w0] = (uint32_t)bg;
      sm.bm_gt[w0 + 1] = (uint32_t)(bg >> 32);
      sm.bm_eq[w0] = (uint32_t)be;
      sm.bm_eq[w0 + 1] = (uint32_t)(be >> 32);
    }
  }
  if (__syncthreads_or(unsafe)) {
    if (tid == 0) count_event(CNT_DECODE_FALLBACK);
    select_row<PICK_NT>(*reinterpret_cast<TopkSmem<PICK_NT>*>(&sm.hist[0][0]), R.src, R.n, k, R.idx, R.sco);
    return;
  }

  // ---- 4. output in slot order (= ascending entry order): the bitmap words
  // are split into Q parts of L slots, thread tid owning part tid % Q of word
  // tid / Q (so the threads hold the slots in order): keys > tau, and the
  // first `need` keys == tau over the whole row ----
  constexpr int NWORDS = PER * PICK_NT / 32;
  constexpr int Q = PICK_NT / NWORDS >= 4 ? 4 : PICK_NT / NWORDS >= 2 ? 2 : 1;
  constexpr int L = 32 / Q;
  constexpr uint32_t LMASK = L == 32 ? 0xFFFFFFFFu : (1u << L) - 1u;
  const int word = tid / Q, wpart = tid % Q;
  const uint32_t wgt = word < NWORDS ? (sm.bm_gt[word] >> (wpart * L)) & LMASK : 0u;
  const uint32_t weq = word < NWORDS ? (sm.bm_eq[word] >> (wpart * L)) & LMASK : 0u;
  const uint32_t pgt = (uint32_t)__popc(wgt), peq = (uint32_t)__popc(weq);
  const uint32_t inc_gt = wave_incl_scan(pgt), inc_eq = wave_incl_scan(peq);
  if (lane == 63) { sm.wv[1][wave] = inc_gt; sm.wv[2][wave] = inc_eq; }
  __syncthreads();
  uint32_t gt_before = inc_gt - pgt, eq_before = inc_eq - peq;
  gt_before += waves_below(sm.wv[1], wave);
  eq_before += waves_below(sm.wv[2], wave);
  uint32_t pos = gt_before + min(eq_before, need);
  uint32_t e_seen = eq_before;
  uint32_t take = wgt;
  for (uint32_t m = weq; m; m &= m - 1) {
    const int bit = __ffs(m) - 1;
    if (e_seen++ < need) take |= 1u << bit;
  }
  const int s0 = word * 32 + wpart * L;
  for (; take; take &= take - 1) {
    const int s = s0 + __ffs(take) - 1;
    if (pos < (uint32_t)k) {
      R.idx[pos] = (int32_t)(s < PICK_STASH ? sm.sel[s] : R.cand[s].y);
      if (R.sco) R.sco[pos] = __uint_as_float(R.cand[s].x);
    }
    ++pos;
  }
}

// One workgroup per row: the row's geometry, then the body specialised for
// its slots per thread (a uniform branch).
__global__ __launch_bounds__(PICK_NT) void long_pick_kernel(IndexerArgs a) {
  __shared__ PickSmem sm;
  PickRow R;
  R.row = blockIdx.x;
  const int b = R.row / a.Tq, t = R.row % a.Tq;
  R.k = a.topk;
  const LongWs L = long_ws(a.ws, a.B * a.Tq, a.Nc_cap);
  R.idx = a.idx_out + (size_t)R.row * R.k;
  R.sco = a.score_out ? a.score_out + (size_t)R.row * R.k : nullptr;
  R.src = reinterpret_cast<const uint32_t*>(L.scores) + (size_t)R.row * nc_pad(a.Nc_cap);
  R.meta = reinterpret_cast<const uint2*>(L.meta) + (size_t)R.row * L.nch;
  R.cand = reinterpret_cast<const uint2*>(L.cand) + (size_t)R.row * L.nch * SCORE_CHUNK;
  R.n = row_len(a, b, t);
  if (R.n <= R.k) {
    write_all_eligible(R.n, R.k, R.src, R.idx, R.sco, PICK_NT);
    return;
  }
  R.nch = (R.n + SCORE_CHUNK - 1) / SCORE_CHUNK;
  R.cap = chunk_cap_n(R.k, R.n);
  R.lg = 31 - __clz(R.cap);                                  // cap is a power of two
  R.nslot = R.nch << R.lg;                                   // <= L.nch * SCORE_CHUNK
  const int per = (R.nslot + PICK_NT - 1) / PICK_NT;
  if (per > PICK_MAXPER || R.nch > PICK_MAXCH) {
    if (threadIdx.x == 0) count_event(CNT_DECODE_FALLBACK);
    select_row<PICK_NT>(*reinterpret_cast<TopkSmem<PICK_NT>*>(&sm.hist[0][0]), R.src, R.n, R.k, R.idx, R.sco);
    return;
  }
  if (per <= 8) pick_body<8>(sm, R);
  else if (per <= 16) pick_body<16>(sm, R);
  else pick_body<PICK_MAXPER>(sm, R);
}

// --------------------------- fused prefill path ----------------------------
// One workgroup (8 waves) per FQ consecutive query tokens.  Scores never reach
// HBM: the eligible indexer keys are streamed twice (from L2) and the scores
// recomputed on MFMA each time.
//   pass 1: an 11-bit radix histogram of each token's score keys in LDS (bits
//           30..20 — bit 31 is the sign, always 0 here — as two 16-bit counters
//           per word); two tokens per wave then find the bin b1 holding the
//           k-th largest key and the count above it;
//   pass 2: entries whose digit is above b1 set their bit in the token's LDS
//           selection bitmap, entries inside b1 append (key, index) to the
//           token's candidate slots;
//   resolve: per token, a radix select over the low 20 bits of the candidates
//           (lowest index among equal keys) marks the remaining winners in the
//           bitmap, which is then written out as the ascending index list.
// A token whose boundary bin overflows its candidate slots is rescored into the
// workspace and selected by the exact block-wide select.
static constexpr int FQ = 16;                  // query tokens per workgroup
static constexpr int FNT = 512;                // threads per workgroup
static constexpr int FNW = FNT / 64;
static constexpr int FK = 512;                 // largest top-k on this path
static constexpr int FCAP = 512;               // boundary-bin candidates per token
static constexpr int FMAXN = 8192;             // largest eligible row on this path
static constexpr int FBM = FMAXN / 32;         // bitmap words per token
// Histogram rows are padded with one word after every 32 (pass 1) or 16
// (resolve) so that the per-lane bin ranges of the top-down scan fall in
// distinct LDS banks.
static constexpr int HROW = 1024 + 1024 / 32;  // pass-1 row: 2048 bins as 16-bit pairs
static constexpr int SROW = 1024 + 1024 / 16;  // resolve row: 1024 bins
__device__ __forceinline__ int hpad(int w) { return w + (w >> 5); }
__device__ __forceinline__ int spad(int w) { return w + (w >> 4); }

struct FusedSmem {
  union {
    uint32_t hist[FQ + 1][HROW];               // bin i: word hpad(i & 1023), half i >> 10;
                                               // row FQ absorbs ineligible entries
    uint32_t cand[FQ][FCAP][2];                // (key, index)
  } u;
  uint32_t bm[FQ][FBM];
  uint32_t scr[FNW][SROW];                     // per-wave radix scratch; fallback select
  uint32_t ncand[FQ], b1[FQ], above[FQ], fb[FQ];
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Wave-level: scanning nb bins from the top down, the bin where the running
// count first reaches `need` (>= 1, <= total) and the count strictly above it.
template <typename Cnt>
__device__ __forceinline__ void wave_find_bin(int nb, uint32_t need, Cnt cnt, uint32_t& bin,
                                              uint32_t& above) {
  const int lane = threadIdx.x & 63;
  const int per = nb / 64;
  const int hi = nb - lane * per;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += cnt(hi - 1 - i);
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t excl = incl - local;
  const bool mine = excl < need && incl >= need;
  uint32_t bb = 0, ab = 0;
  if (mine) {
    uint32_t cum = excl;
    for (int i = 0; i < per; ++i) {
      const uint32_t h = cnt(hi - 1 - i);
      if (cum + h >= need) { bb = hi - 1 - i; ab = cum; break; }
      cum += h;
    }
  }
  const uint64_t m = __ballot(mine);
  const int src = m ? __ffsll((unsigned long long)m) - 1 : 0;
  bin = (uint32_t)__builtin_amdgcn_readlane((int)bb, src);
  above = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
}

template <int QK, int DI, int HI>
__global__ __launch_bounds__(FNT) void fused_prefill_kernel(IndexerArgs a) {
  constexpr int KC = DI / 32;
  constexpr int NRT = HI;                      // 16-row tiles of (token, head) rows
  constexpr int SPL = 4 / HI;                  // scores per lane per row tile
  constexpr int TPW = FQ / FNW;                // tokens resolved per wave
  using F = typename QkTraits<QK>::F;
  extern __shared__ __align__(16) unsigned char fsm_raw[];
  FusedSmem& sm = *reinterpret_cast<FusedSmem*>(fsm_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int b = blockIdx.y, t0 = blockIdx.x * FQ;
  const int nt = min(FQ, a.Tq - t0);
  const int k = a.topk;
  const int ne_max = row_len(a, b, t0 + nt - 1);
  const size_t rb = qk_row_bytes<QK>(DI);

  // A operands: row 16 rt + r of the tiles is token (16 rt + r) / HI, head (16 rt + r) % HI
  F qa[NRT][KC];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int tt = (16 * rt + r) / HI, h = (16 * rt + r) % HI;
    const size_t qrow = ((size_t)b * a.Tq + t0 + tt) * HI + h;
    const char* qptr = reinterpret_cast<const char*>(a.qi) + qrow * rb;
    const uint8_t* qsc = QK == QK_FP4 ? reinterpret_cast<const uint8_t*>(a.qi_scale) + qrow * (DI / 32) : nullptr;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (tt < nt) load_qk_frag<QK>(qa[rt][c], qptr, qsc, 8 * (g * KC + c));
      else frag_zero(qa[rt][c]);
    }
  }
  // accumulator rows of lane group g in tile rt: 16 rt + 4g + i -> token (16 rt + 4g + i) / HI
  float wr[NRT][4];
  int tok[NRT][SPL], tne[NRT][SPL];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * rt + 4 * g + i;
      const int tt = rr / HI, h = rr % HI;
      float wv = 0.f;
      if (tt < nt) {
        const size_t wi = ((size_t)b * a.Tq + t0 + tt) * HI + h;
        wv = a.w[wi];
        if constexpr (QK == QK_FP8) wv *= reinterpret_cast<const float*>(a.qi_scale)[wi];
      }
      wr[rt][i] = wv;
    }
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp) {
      const int tt = (16 * rt + 4 * g) / HI + sp;
      tok[rt][sp] = tt;
      tne[rt][sp] = tt < nt ? row_len(a, b, t0 + tt) : 0;
    }
  }
  for (int i = tid; i < (FQ + 1) * HROW; i += FNT) (&sm.u.hist[0][0])[i] = 0u;
  for (int i = tid; i < FQ * FBM; i += FNT) (&sm.bm[0][0])[i] = 0u;
  if (tid < FQ) { sm.ncand[tid] = 0; sm.fb[tid] = 0; sm.b1[tid] = 0; sm.above[tid] = 0; }
  __syncthreads();

  const char* kbase = reinterpret_cast<const char*>(a.kic) + (size_t)b * a.Nc_cap * rb;
  const uint8_t* sbase = QK == QK_FP4 ? reinterpret_cast<const uint8_t*>(a.kic_scale) + (size_t)b * a.Nc_cap * (DI / 32) : nullptr;
  const float* fsc = QK == QK_FP8 ? reinterpret_cast<const float*>(a.kic_scale) + (size_t)b * a.Nc_cap : nullptr;

  // Scores of entries e0 + 16 wave + r (e0 steps by 16 FNW) for every row tile;
  // f(rt, sp, entry, key, eligible) is called for each.  All MFMAs of an entry
  // tile issue before the epilogue reads their results.
  auto pass = [&](auto&& f) {
    RawFrag<QK> kb[KC];
    float ks = 1.f;
    auto load = [&](int e0) {
      const int e = min(e0 + 16 * wave + r, ne_max - 1);
#pragma unroll
      for (int c = 0; c < KC; ++c)
        load_raw<QK>(kb[c], kbase + (size_t)e * rb, QK == QK_FP4 ? sbase + (size_t)e * (DI / 32) : nullptr,
                     8 * (g * KC + c));
      if constexpr (QK == QK_FP8) ks = fsc[e];
    };
    if (ne_max > 0) load(0);
#pragma unroll 1
    for (int e0 = 0; e0 < ne_max; e0 += 16 * FNW) {
      RawFrag<QK> cur[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) cur[c] = kb[c];
      const float cks = ks;
      if (e0 + 16 * FNW < ne_max) load(e0 + 16 * FNW);
      const int e = e0 + 16 * wave + r;
      f32x4 acc[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) mma16(acc[rt], qa[rt][c], widen<QK>(cur[c]));
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
        for (int sp = 0; sp < SPL; ++sp) {
          // scores are sums of non-negative terms starting from +0, so never -0
          float sc = 0.f;
#pragma unroll
          for (int h = 0; h < HI; ++h) {
            const float x = __int_as_float(max(__float_as_int(acc[rt][sp * HI + h]), 0));   // ReLU
            sc = fmaf(wr[rt][sp * HI + h], x, sc);
          }
          if constexpr (QK == QK_FP8) sc *= cks;
          f(rt, sp, e, __float_as_uint(sc), e < tne[rt][sp]);
        }
      }
    }
  };

  // ---- pass 1: per-token histograms of key bits 30..20 ----
  pass([&](int rt, int sp, int e, uint32_t key, bool ok) {
    const uint32_t bin = key >> 20;
    atomicAdd(&sm.u.hist[ok ? tok[rt][sp] : FQ][hpad(bin & 1023u)], 1u << ((bin >> 10) << 4));
  });
  __syncthreads();
  for (int j = 0; j < TPW; ++j) {
    const int tt = TPW * wave + j;
    if (tt >= nt || row_len(a, b, t0 + tt) <= k) continue;
    const uint32_t* hrow = sm.u.hist[tt];
    uint32_t bin, ab;
    wave_find_bin(2048, (uint32_t)k,
                  [&](int i) { return (hrow[hpad(i & 1023)] >> ((i >> 10) << 4)) & 0xFFFFu; }, bin, ab);
    if (lane == 0) { sm.b1[tt] = bin; sm.above[tt] = ab; }
  }
  __syncthreads();
  uint32_t tb1[NRT][SPL];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int sp = 0; sp < SPL; ++sp) tb1[rt][sp] = tne[rt][sp] > k ? sm.b1[tok[rt][sp]] : 0xFFFFFFFFu;
  __syncthreads();                                           // histograms become candidate slots
  // ---- pass 2: bits above b1, candidates inside b1 ----
  pass([&](int rt, int sp, int e, uint32_t key, bool ok) {
    const uint32_t d = key >> 20;
    if (ok && d >= tb1[rt][sp]) {
      const int tt = tok[rt][sp];
      if (d > tb1[rt][sp]) {
        atomicOr(&sm.bm[tt][e >> 5], 1u << (e & 31));
      } else {
        const uint32_t slot = atomicAdd(&sm.ncand[tt], 1u);
        if (slot < (uint32_t)FCAP) { sm.u.cand[tt][slot][0] = key; sm.u.cand[tt][slot][1] = (uint32_t)e; }
      }
    }
  });
  __syncthreads();
  // ---- resolve the boundary bin, write ascending lists ----
  uint32_t* scr = sm.scr[wave];
  for (int j = 0; j < TPW; ++j) {
    const int tt = TPW * wave + j;
    if (tt >= nt) break;
    const int ne = row_len(a, b, t0 + tt);
    int32_t* idx = a.idx_out + ((size_t)b * a.Tq + t0 + tt) * k;
    if (ne <= k) {
      for (int i = lane; i < k; i += 64) idx[i] = i < ne ? i : -1;
      continue;
    }
    const uint32_t ncand = sm.ncand[tt];
    uint32_t rem = (uint32_t)k - sm.above[tt];
    if (ncand > (uint32_t)FCAP || rem > ncand) {
      if (lane == 0) {
        sm.fb[tt] = 1u;
        count_event(CNT_PREFILL_FALLBACK);
      }
      continue;
    }
    const uint32_t(*cand)[2] = sm.u.cand[tt];
    uint32_t prefix = 0, pmask = 0;
    for (int p = 0; p < 2; ++p) {
      const int sh = p == 0 ? 10 : 0;
      for (int i = lane; i < SROW; i += 64) scr[i] = 0u;
      wave_sync();
      for (uint32_t i = lane; i < ncand; i += 64) {
        const uint32_t low = cand[i][0] & 0xFFFFFu;
        if ((low & pmask) == prefix) atomicAdd(&scr[spad((low >> sh) & 1023u)], 1u);
      }
      wave_sync();
      uint32_t bin, ab;
      wave_find_bin(1024, rem, [&](int i) { return scr[spad(i)]; }, bin, ab);
      prefix |= bin << sh;
      pmask |= 1023u << sh;
      rem -= ab;
      wave_sync();
    }
    // rem keys equal to the threshold's low bits remain to be taken
    uint32_t neq = 0;
    for (uint32_t i = lane; i < ncand; i += 64) neq += (cand[i][0] & 0xFFFFFu) == prefix;
    neq = (uint32_t)wave_sum((float)neq);
    for (uint32_t i = lane; i < ncand; i += 64) {
      const uint32_t low = cand[i][0] & 0xFFFFFu;
      bool take = low > prefix;
      if (low == prefix) {
        if (neq == rem) {
          take = true;
        } else {
          uint32_t rank = 0;
          for (uint32_t q = 0; q < ncand; ++q)
            rank += ((cand[q][0] & 0xFFFFFu) == prefix) && (cand[q][1] < cand[i][1]);
          take = rank < rem;
        }
      }
      if (take) atomicOr(&sm.bm[tt][cand[i][1] >> 5], 1u << (cand[i][1] & 31));
    }
    wave_sync();
    constexpr int WPL = FBM / 64;                           // bitmap words per lane
    const int nw = (ne + 31) / 32;
    uint32_t words[WPL];
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < WPL; ++q) {
      const int w = lane * WPL + q;
      words[q] = w < nw ? sm.bm[tt][w] : 0u;
      cnt += (uint32_t)__popc(words[q]);
    }
    uint32_t pos = wave_incl_scan(cnt) - cnt;
#pragma unroll
    for (int q = 0; q < WPL; ++q) {
      uint32_t word = words[q];
      while (word) {
        const int bit = __ffs(word) - 1;
        word &= word - 1;
        if (pos < (uint32_t)k) idx[pos] = (lane * WPL + q) * 32 + bit;
        ++pos;
      }
    }
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)pos, 63);
    for (uint32_t i = tot + lane; i < (uint32_t)k; i += 64) idx[i] = -1;
    wave_sync();
  }
  __syncthreads();
  // ---- exact fallback for tokens whose boundary bin overflowed ----
  for (int tt = 0; tt < nt; ++tt) {
    if (!sm.fb[tt]) continue;                                // uniform: LDS after a barrier
    const int ne = row_len(a, b, t0 + tt);
    float* srow = reinterpret_cast<float*>(a.ws) + ((size_t)b * a.Tq + t0 + tt) * nc_pad(a.Nc_cap);
    pass([&](int rt, int sp, int e, uint32_t key, bool ok) {
      if (ok && tok[rt][sp] == tt) srow[e] = __uint_as_float(key);
    });
    __syncthreads();
    TopkSmem<FNT>& ts = *reinterpret_cast<TopkSmem<FNT>*>(&sm.scr[0][0]);
    select_row<FNT>(ts, reinterpret_cast<const uint32_t*>(srow), ne, k,
                    a.idx_out + ((size_t)b * a.Tq + t0 + tt) * k, nullptr);
    __syncthreads();
  }
}

static bool use_fused_prefill(const IndexerArgs& a) {
  return a.Tq > 4 && a.topk <= FK && a.Nc_cap <= FMAXN && a.score_out == nullptr;
}

template <int QK, int DI, int HI>
static hipError_t launch_fused(const IndexerArgs& a, hipStream_t st) {
  const size_t lds = sizeof(FusedSmem);
  auto kfn = fused_prefill_kernel<QK, DI, HI>;
  hipError_t e = ensure_lds_limit((const void*)kfn, lds);
  if (e != hipSuccess) return e;
  ProfScope ps("indexer_fused", st);
  hipLaunchKernelGGL(kfn, dim3((a.Tq + FQ - 1) / FQ, a.B), dim3(FNT), lds, st, a);
  return hipGetLastError();
}

template <int QK, int DI>
static hipError_t launch_fused_hi(const IndexerArgs& a, hipStream_t st) {
  if (a.HI == 1) return launch_fused<QK, DI, 1>(a, st);
  if (a.HI == 2) return launch_fused<QK, DI, 2>(a, st);
  return launch_fused<QK, DI, 4>(a, st);
}

template <int QK>
static hipError_t launch_fused_di(const IndexerArgs& a, hipStream_t st) {
  return a.dI == 32 ? launch_fused_hi<QK, 32>(a, st) : launch_fused_hi<QK, 64>(a, st);
}

hipError_t counter_read(int which, unsigned long long* value, bool reset) {
  unsigned long long v[CNT_COUNT];
  hipError_t e = hipMemcpyFromSymbol(v, HIP_SYMBOL(g_counters), sizeof(v), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *value = v[which];
  if (!reset) return hipSuccess;
  v[which] = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_counters), v, sizeof(v), 0, hipMemcpyHostToDevice);
}

// --------------------------------- launch ----------------------------------
size_t indexer_workspace(int B, int Tq, int Nc_cap, int HI, int dI, int topk, int qk) {
  (void)HI; (void)dI; (void)qk;
  if (use_long_path(Tq, Nc_cap)) return long_ws_bytes(B * Tq, Nc_cap);
  return (size_t)B * Tq * nc_pad(Nc_cap) * sizeof(float);
}

template <int QK, int DI, int HI>
static void launch_scores(const IndexerArgs& a, hipStream_t st, bool long_path) {
  const int ne_ub = std::min((a.max_pos + 1) / a.m, a.Nc_cap);
  if (ne_ub <= 0) return;
  if (long_path) {
    const int nch = (ne_ub + SCORE_CHUNK - 1) / SCORE_CHUNK;
    ProfScope ps("indexer_score", st);
    if constexpr (QK == QK_FP4 && HI == 4)
      hipLaunchKernelGGL((score_row_fp4_kernel<DI>), dim3(nch * a.B * a.Tq), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((score_row_kernel<QK, DI, HI>), dim3((nch + SCORE_CPW - 1) / SCORE_CPW * a.B * a.Tq),
                         dim3(256), 0, st, a);
  } else {
    const int TT = 16 / HI;
    dim3 grid((ne_ub + SCORE_WG_ENTRIES - 1) / SCORE_WG_ENTRIES, (a.Tq + TT - 1) / TT, a.B);
    ProfScope ps("indexer_score", st);
    hipLaunchKernelGGL((score_tile_kernel<QK, DI, HI>), grid, dim3(256), 0, st, a);
  }
}

template <int QK, int DI>
static void launch_scores_hi(const IndexerArgs& a, hipStream_t st, bool lp) {
  if (a.HI == 1) launch_scores<QK, DI, 1>(a, st, lp);
  else if (a.HI == 2) launch_scores<QK, DI, 2>(a, st, lp);
  else launch_scores<QK, DI, 4>(a, st, lp);
}

template <int QK>
static void launch_scores_di(const IndexerArgs& a, hipStream_t st, bool lp) {
  if (a.dI == 32) launch_scores_hi<QK, 32>(a, st, lp);
  else launch_scores_hi<QK, 64>(a, st, lp);
}

hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t st) {
  if (a.B == 0 || a.Tq == 0) return hipSuccess;
  if (use_fused_prefill(a)) {
    switch (a.qk) {
      case QK_F32: return launch_fused_di<QK_F32>(a, st);
      case QK_BF16: return launch_fused_di<QK_BF16>(a, st);
      case QK_FP8: return launch_fused_di<QK_FP8>(a, st);
      case QK_FP4: return launch_fused_di<QK_FP4>(a, st);
    }
  }
  const bool lp = use_long_path(a.Tq, a.Nc_cap);
  switch (a.qk) {
    case QK_F32: launch_scores_di<QK_F32>(a, st, lp); break;
    case QK_BF16: launch_scores_di<QK_BF16>(a, st, lp); break;
    case QK_FP8: launch_scores_di<QK_FP8>(a, st, lp); break;
    case QK_FP4: launch_scores_di<QK_FP4>(a, st, lp); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ProfScope ps("indexer_topk", st);
  if (lp) hipLaunchKernelGGL(long_pick_kernel, dim3(a.B * a.Tq), dim3(PICK_NT), 0, st, a);
  else hipLaunchKernelGGL(topk_row_kernel, dim3(a.Tq, a.B), dim3(TOPK_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
