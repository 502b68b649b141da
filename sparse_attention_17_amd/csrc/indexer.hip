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
#include "pick_impl.hpp"

#include <map>
#include <mutex>

namespace csa {

// Event counters for measurement tools (csa_profile_counter): rows whose
// top-k took the exact fallback select.  Incremented by one lane per event.
__device__ unsigned long long g_counters[CNT_COUNT];

__device__ __forceinline__ void count_event(int which) {
  atomicAdd(&g_counters[which], 1ull);
}

static constexpr int SCORE_WG_ENTRIES = 256;   // prefill tile kernel: 4 waves x 4 tiles x 16
static constexpr int SCORE_CPW = 1;            // chunks per score_row_kernel workgroup
static constexpr int SCORE_DEPTH = 3;          // entry groups in flight per wave

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

static bool use_long_path(int Tq, int Nc_cap) { return Tq <= 4 && Nc_cap > TOPK_LDS_KEYS; }

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
  // FP8 codes are widened exactly to bf16 and multiplied on the bf16 MFMA,
  // which accumulates in fp32; the native FP8 MFMA was measured on gfx950 at
  // ~1e-5 relative error in these sums, outside the 1e-6 near-tie band.
  F qv[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) load_qk_frag<QK>(qv[c], qptr, qsc, 8 * (g * KC + c));
  F qa[TPC][KC];
#pragma unroll
  for (int u = 0; u < TPC; ++u)
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (u == uq) qa[u][c] = qv[c];
      else frag_zero(qa[u][c]);
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
      for (int c = 0; c < KC; ++c) mma16(acc, qa[u][c], widen<QK>(cur[u][c]));
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
        // written once, read back only by a second pick round: streamed
        // past the caches
        __builtin_nontemporal_store(sc, srow + e);
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
      __builtin_nontemporal_store(sc, srow + e);
      sk[e - c0] = __float_as_uint(sc);
      atomicAdd(&hist[__float_as_uint(sc) >> (32 - H1_BITS)], 1u);
    }
  };
  // The chunk's groups of this wave (64 entries each, 256 apart) are all
  // requested up front — unconditionally, addresses clamped to the last
  // entry — and then scored in order: every load is in flight before the
  // first wait, and a fixed load count keeps the wait counts exact.
  constexpr int STRIDE = 4 * EPC;
  constexpr int NGW = SCORE_CHUNK / STRIDE;
  u32x4 kv[NGW][NM];
  int ks[NGW][NM];
  const int e0 = c0 + wave * EPC;
#pragma unroll
  for (int gi = 0; gi < NGW; ++gi) load_group(e0 + gi * STRIDE, kv[gi], ks[gi]);
#pragma unroll
  for (int gi = 0; gi < NGW; ++gi)
    if (e0 + gi * STRIDE < c1) process(e0 + gi * STRIDE, kv[gi], ks[gi]);   // uniform
  __syncthreads();
  if (n > a.topk) chunk_cut(a, L, row, chunk, n, c0, c1 - c0, sk, hist, cut_ws);
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
// One 1024-thread workgroup per query row picks the row's k largest keys among
// the chunks' candidates (pick_row).
__global__ __launch_bounds__(1024) void long_pick_kernel(IndexerArgs a) {
  __shared__ PickSmem<1024> sm;
  pick_row<1024>(sm, a, blockIdx.x, g_counters);
}

// --------------------------- fused prefill path ----------------------------
// One workgroup (8 waves) per FQ consecutive query tokens.  Scores never reach
// HBM; the eligible indexer keys stream from L2 and the scores are computed on
// MFMA.  Workgroups are launched longest rows first (causal rows grow with the
// token), so the last workgroups to start are the shortest.
//   sample: the scores of one 128-entry step in every FSAMPLE (a block-strided
//           quarter of the row) feed an 11-bit radix histogram per token in
//           LDS (key bits 30..20 — bit 31, the sign, is always 0 here — as two
//           16-bit counters per word).  From it each token takes a band of
//           digits [b_lo, b_hi] meant to hold its k-th largest score: b_hi
//           leaves about (k - 3 sigma) sampled scores above it, b_lo about
//           (k + 3 sigma) at or above it, sigma the binomial spread of the
//           sample count above the k-th largest score; inside each of those
//           two digits the band edge is placed by linear interpolation of the
//           digit's key range over its sampled count;
//   full pass: every score is computed once; the ballot of "above the band"
//           over a wave holds four tokens' 16-entry bitmap fields and is
//           stored whole by one lane (one writer per field: no atomics, no
//           clearing); scores inside the band are appended as (key, entry)
//           records to the wave's stream of the lane's half of the ballot
//           (two tokens), placed by wave-uniform counters and the lane's rank
//           in the ballot;
//   resolve: one wave per stream set (two tokens: the same half of one
//           unit's ballots in every wave).  The band holds the k-th largest
//           score exactly when the entries above it number at most k and
//           those above plus inside it at least k (every dropped entry is
//           below every kept one; checked).  A 128-bin histogram of each
//           token's records over its band range (both tokens in one pass)
//           gives the bin of the k-th largest key; records above it are
//           selected, and those of that bin (up to 64) ranked exactly —
//           larger key first, then lower index; a bin holding more is
//           histogrammed again over its own range, down to single keys,
//           whose ties go to the lowest indices.  The bitmap is written out
//           as the ascending index list.
// The LDS footprint stays under half a CU's, so two workgroups share a CU and
// one's band resolve overlaps the other's scoring.
// A token whose band misses, or whose stream set overflows, is rescored into
// the workspace and selected by the exact block-wide select.
static constexpr int FQ = 16;                  // query tokens per workgroup
static constexpr int FNT = 512;                // threads per workgroup
static constexpr int FNW = FNT / 64;
static constexpr int FK = 512;                 // largest top-k on this path
static constexpr int FMAXN = 8192;             // largest eligible row on this path
static constexpr int FG = FMAXN / 16;          // 16-entry groups per row
static constexpr int FU = 4;                   // ballot units (row tile, score slot) of 4 tokens
static constexpr int FCAPH = 108;              // band records per (unit, wave, half) stream
static constexpr int FSTEP = 16 * FNW;         // entries per step of the scoring loop
static constexpr int FSAMPLE = 4;              // one step in FSAMPLE is sampled
// Histogram rows are padded with one word after every 32 (sample) or 16
// (resolve) so that the per-lane bin ranges of the top-down scan fall in
// distinct LDS banks.
static constexpr int HROW = 1024 + 1024 / 32;  // sample row: 2048 bins as 16-bit pairs
static constexpr int SROW = 2 * (128 + 128 / 16);   // resolve row: two tokens' 128 bins
__device__ __forceinline__ int hpad(int w) { return w + (w >> 5); }
__device__ __forceinline__ int spad(int w) { return w + (w >> 4); }

// The sample histograms are dead once the bands are known, so the record
// streams and the selection bitmaps share their space; the whole stays
// under half of a CU's LDS, so two workgroups share a CU and one's resolve
// overlaps the other's scoring.
struct FusedSmem {
  union {
    uint32_t hist[FQ + 1][HROW];               // bin i: word hpad(i & 1023), half i >> 10;
                                               // row FQ absorbs ineligible entries
    struct {
      uint32_t cand[FU][2][FNW][FCAPH][2];     // (key, entry | g << 16) per (unit, g >> 1, wave)
      uint64_t bm[FG][FU];                     // 16-bit field g: entries 16E.. of token (u, g)
    } s;
  } u;
  uint32_t scr[FNW][SROW];                     // per-wave resolve scratch; fallback select
  uint32_t ncs[FU][FNW][2];                    // records per (unit, wave, half)
  uint32_t lo_key[FQ], hi_key[FQ], fb[FQ];
};
static_assert(sizeof(FusedSmem) <= 80 * 1024, "two workgroups per CU");

// Token of lane group g (lanes 16g..16g+15) in ballot unit u: accumulator rows
// 16 rt + 4g + i hold token (16 rt + 4g + i) / HI, head (16 rt + 4g + i) % HI;
// unit u = rt * (4 / HI) + sp takes the sp-th token of the lane's four rows.
template <int HI>
__device__ __forceinline__ int unit_token(int u, int g) {
  constexpr int SPL = 4 / HI;
  return (16 * (u / SPL) + 4 * g) / HI + u % SPL;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave-level: with every lane holding the summed count `local` of its run of
// `per` bins (lane 0 the top run), the bin where the running count from the
// top first reaches `need` (>= 1, <= total) and the count strictly above it.
// The run is found by a scan; its bins are then read one per lane (cnt(i) for
// bin i of nb) and scanned again (no serial search).
template <typename Cnt>
__device__ __forceinline__ void wave_find_bin_runs(int nb, int per, uint32_t incl, uint32_t local,
                                                   uint32_t need, Cnt cnt, uint32_t& bin,
                                                   uint32_t& above) {
  const int lane = threadIdx.x & 63;
  const uint32_t excl = incl - local;
  const uint64_t m = __ballot(excl < need && incl >= need);
  const int src = m ? __ffsll((unsigned long long)m) - 1 : 0;
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)excl, src);
  const int shi = nb - src * per;                            // lane src's bins: shi-per .. shi-1
  const uint32_t h = lane < per ? cnt(shi - 1 - lane) : 0u;
  const uint32_t hin = wave_incl_scan(h);
  const uint64_t m2 = __ballot(lane < per && base + hin >= need);
  const int f = m2 ? __ffsll((unsigned long long)m2) - 1 : 0;
  bin = (uint32_t)(shi - 1 - f);
  above = base + (uint32_t)__builtin_amdgcn_readlane((int)(hin - h), f);
}
template <typename Cnt>
__device__ __forceinline__ void wave_find_bin(int nb, uint32_t need, Cnt cnt, uint32_t& bin,
                                              uint32_t& above) {
  const int lane = threadIdx.x & 63;
  const int per = nb / 64;
  const int hi = nb - lane * per;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += cnt(hi - 1 - i);
  wave_find_bin_runs(nb, per, wave_incl_scan(local), local, need, cnt, bin, above);
}

// Sampled entries of a row of n eligible entries: the first 128 of every
// FSAMPLE * 128 (the steps the sample pass scores).
__device__ __forceinline__ int sample_count(int n) {
  const int blk = FSAMPLE * FSTEP;
  return (n / blk) * FSTEP + min(n % blk, FSTEP);
}

template <int QK, int DI, int HI>
__global__ __launch_bounds__(FNT, 4) void fused_prefill_kernel(IndexerArgs a) {
  constexpr int KC = DI / 32;
  constexpr int NRT = HI;                      // 16-row tiles of (token, head) rows
  constexpr int SPL = 4 / HI;                  // scores per lane per row tile
  constexpr int TPW = FQ / FNW;                // tokens per wave in the band and resolve phases
  static_assert(NRT * SPL == FU, "four ballot units");
  using F = typename QkTraits<QK>::F;
  extern __shared__ __align__(16) unsigned char fsm_raw[];
  FusedSmem& sm = *reinterpret_cast<FusedSmem*>(fsm_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int b = blockIdx.y, t0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * FQ;
  const int nt = min(FQ, a.Tq - t0);
  const int k = a.topk;
  const int ne_max = row_len(a, b, t0 + nt - 1);
  const int ne_min = row_len(a, b, t0);                      // rows grow with the token
  const size_t rb = qk_row_bytes<QK>(DI);

  // Scoring operands (loaded again for the rare exact fallback rather than
  // held in registers through the resolve).  A operands: row 16 rt + r of
  // the tiles is token (16 rt + r) / HI, head (16 rt + r) % HI; the
  // accumulator rows of lane group g in tile rt are 16 rt + 4g + i.
  F qa[NRT][KC];
  float wr[NRT][4];
  int tok[FU], tne[FU];
  auto load_operands = [&]() {
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
    }
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      tok[u] = unit_token<HI>(u, g);
      tne[u] = tok[u] < nt ? row_len(a, b, t0 + tok[u]) : 0;
    }
  };
  load_operands();
  static_assert((FQ + 1) * HROW % 4 == 0, "histograms cleared 16 bytes at a time");
  for (int i = tid; i < (FQ + 1) * HROW / 4; i += FNT) reinterpret_cast<uint4*>(&sm.u.hist[0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < FQ) sm.fb[tid] = 0;
  __syncthreads();

  const char* kbase = reinterpret_cast<const char*>(a.kic) + (size_t)b * a.Nc_cap * rb;
  const uint8_t* sbase = QK == QK_FP4 ? reinterpret_cast<const uint8_t*>(a.kic_scale) + (size_t)b * a.Nc_cap * (DI / 32) : nullptr;
  const float* fsc = QK == QK_FP8 ? reinterpret_cast<const float*>(a.kic_scale) + (size_t)b * a.Nc_cap : nullptr;

  // Scores of entries e0 + 16 wave + r for e0 = first, first + stride, ...
  // (< ne_max); f(u, e, score, valid, e0) is called for each ballot unit,
  // valid = the entry is eligible for the lane's token (checked only in the
  // steps that reach past the shortest row).  All MFMAs of an entry tile
  // issue before the epilogue reads them.  Two key buffers rotate: each is
  // reloaded right after its step has read it, so the next step's loads are
  // in flight during each step's compute (the keys come from L2), and no
  // in-flight load result is ever copied between registers (a copy would
  // have to wait for it).  A third buffer pushed the kernel past its 128
  // registers: its spill reloads, which share the vector-memory counter with
  // the key loads, then waited for every prefetch in flight.
  auto pass = [&](int first, int stride, auto&& f) {
    RawFrag<QK> kb0[KC], kb1[KC];
    float ks0 = 1.f, ks1 = 1.f;
    // Loads are issued unconditionally (clamped to the last eligible entry):
    // with a fixed number of loads per step the compiler's wait counts stay
    // exact across the loop's back edge.
    auto load = [&](RawFrag<QK> (&kb)[KC], float& ks, int e0) {
      const int e = min(e0 + 16 * wave + r, ne_max - 1);
#pragma unroll
      for (int c = 0; c < KC; ++c)
        load_raw<QK>(kb[c], kbase + (size_t)e * rb, QK == QK_FP4 ? sbase + (size_t)e * (DI / 32) : nullptr,
                     8 * (g * KC + c));
      if constexpr (QK == QK_FP8) ks = fsc[e];
    };
    auto step = [&](auto full, int e0, const RawFrag<QK> (&cur)[KC], float cks) {
      constexpr bool FULL = decltype(full)::value;
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
          const int u = rt * SPL + sp;
          f(u, e, sc, FULL || e < tne[u], e0);
        }
      }
    };
    auto run = [&](int e0, const RawFrag<QK> (&cur)[KC], float cks) {
      if (e0 + FSTEP <= ne_min) step(std::true_type{}, e0, cur, cks);    // uniform
      else step(std::false_type{}, e0, cur, cks);
    };
    if (first >= ne_max) return;                               // uniform; also ne_max >= 1 below
    load(kb0, ks0, first);
    load(kb1, ks1, first + stride);
#pragma unroll 1
    for (int e0 = first; e0 < ne_max; e0 += 2 * stride) {
      run(e0, kb0, ks0);
      load(kb0, ks0, e0 + 2 * stride);
      if (e0 + stride >= ne_max) break;                       // uniform
      run(e0 + stride, kb1, ks1);
      load(kb1, ks1, e0 + 3 * stride);
    }
  };

  // ---- sample: per-token histograms of key bits 30..20 over a quarter of the row ----
  pass(0, FSAMPLE * FSTEP, [&](int u, int, float sc, bool valid, int) {
    const uint32_t bin = __float_as_uint(sc) >> 20;
    atomicAdd(&sm.u.hist[valid ? tok[u] : FQ][hpad(bin & 1023u)], 1u << ((bin >> 10) << 4));
  });
  __syncthreads();
  // ---- each token's band from its sample ----
  for (int j = 0; j < TPW; ++j) {
    const int tt = TPW * wave + j;
    if (tt >= nt) continue;
    const int ne = row_len(a, b, t0 + tt);
    uint32_t lo_key = 0x7F800000u, hi_key = 0x7F800000u;         // n_e <= k: nothing to select
    if (ne > k) {
      const uint32_t* hrow = sm.u.hist[tt];
      // lane L's run: bins 2047 - 32 L down to 2016 - 32 L, the upper halves
      // (lanes < 32) or lower halves (lanes >= 32) of 32 consecutive words
      const int wb = 992 - 32 * (lane & 31), hs = lane < 32 ? 16 : 0;
      uint32_t local = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) local += (hrow[hpad(wb + i)] >> hs) & 0xFFFFu;
      const uint32_t incl = wave_incl_scan(local);
      auto cnt = [&](int i) { return (hrow[hpad(i & 1023)] >> ((i >> 10) << 4)) & 0xFFFFu; };
      const int ns = sample_count(ne);
      const float p = (float)k / (float)ne;
      const float mean = (float)ns * p;
      const float dev = ceilf(3.f * sqrtf(mean * (1.f - p))) + 2.f;
      const int r_hi = (int)floorf(mean - dev), r_lo = (int)ceilf(mean + dev);
      // Inside the digit that holds the wanted sampled rank, the band edge is
      // placed by linear interpolation of the digit's key range over its
      // sampled count (an estimate: the band is checked exactly later).
      lo_key = 0u;
      if (r_hi >= 1) {                                         // <= r_hi sampled at or above hi_key
        uint32_t bin, ab;
        wave_find_bin_runs(2048, 32, incl, local, (uint32_t)r_hi + 1u, cnt, bin, ab);
        const uint32_t c = cnt((int)bin), top = (bin + 1u) << 20;
        const uint32_t cut = (uint32_t)r_hi > ab
            ? min((uint32_t)ceilf((float)((uint32_t)r_hi - ab) / (float)c * 1048576.f), 1u << 20) : 0u;
        hi_key = min(top - cut, 0x7F800000u);
      }
      if (r_lo <= ns) {                                        // >= r_lo sampled at or above lo_key
        uint32_t bin, ab;
        wave_find_bin_runs(2048, 32, incl, local, (uint32_t)r_lo, cnt, bin, ab);
        const uint32_t c = cnt((int)bin), top = (bin + 1u) << 20;
        lo_key = top - min((uint32_t)ceilf((float)((uint32_t)r_lo - ab) / (float)c * 1048576.f), 1u << 20);
      }
      lo_key = min(lo_key, hi_key);
    }
    if (lane == 0) { sm.lo_key[tt] = lo_key; sm.hi_key[tt] = hi_key; }
  }
  __syncthreads();
  float thr_lo[FU], thr_hi[FU];
#pragma unroll
  for (int u = 0; u < FU; ++u) {
    const bool live = tok[u] < nt;
    thr_lo[u] = __uint_as_float(live ? sm.lo_key[tok[u]] : 0x7F800000u);
    thr_hi[u] = __uint_as_float(live ? sm.hi_key[tok[u]] : 0x7F800000u);
  }
  __syncthreads();                                           // the histograms become record streams
  // ---- full pass: bitmap fields above the band, records inside it ----
  // record counters per (unit, half of the ballot: lanes 0-31 hold token
  // slots 0 and 1, lanes 32-63 slots 2 and 3)
  uint32_t ncnt[FU][2];
#pragma unroll
  for (int u = 0; u < FU; ++u) ncnt[u][0] = ncnt[u][1] = 0;
  const uint32_t gtag = (uint32_t)g << 16;
  const int half = lane >> 5;
  pass(0, FSTEP, [&](int u, int e, float sc, bool valid, int e0) {
    const bool ge_lo = valid && sc >= thr_lo[u];
    const bool ge_hi = valid && sc >= thr_hi[u];
    const uint64_t mhi = __ballot(ge_hi);
    const uint64_t mc = __ballot(ge_lo) & ~mhi;
    if (lane == 0) sm.u.s.bm[(e0 >> 4) + wave][u] = mhi;
    if (mc) {                                                 // uniform
      const uint32_t plo = (uint32_t)__popc((uint32_t)mc), phi = (uint32_t)__popc((uint32_t)(mc >> 32));
      const uint32_t slot = (half ? ncnt[u][1] - plo : ncnt[u][0]) + lanes_below(mc);
      if (ge_lo && !ge_hi && slot < (uint32_t)FCAPH)
        *reinterpret_cast<uint2*>(&sm.u.s.cand[u][half][wave][slot][0]) = make_uint2(__float_as_uint(sc), (uint32_t)e | gtag);
      ncnt[u][0] += plo;
      ncnt[u][1] += phi;
    }
  });
  if (lane < 2 * FU) {
#pragma unroll
    for (int u = 0; u < FU; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (lane == 2 * u + h) sm.ncs[u][wave][h] = ncnt[u][h];
  }
  __syncthreads();
  // ---- resolve the bands of the wave's two tokens, write ascending lists ----
  {
    const int u = wave >> 1, hf = wave & 1, g0 = 2 * hf;
    const uint32_t cs = lane < FNW ? sm.ncs[u][lane][hf] : 0u;
    const bool sovf = wave_max_u32(cs) > (uint32_t)FCAPH;
    const uint32_t nrec = min(cs, (uint32_t)FCAPH);
    const uint16_t* bm16 = reinterpret_cast<const uint16_t*>(&sm.u.s.bm[0][0]);
    uint32_t* bm32 = reinterpret_cast<uint32_t*>(&sm.u.s.bm[0][0]);
    // f(ok, j, key, entry) over the records of the stream set with every lane
    // active (so f may take ballots); ok: the lane holds a record, of token
    // slot g0 + j.  A stream's slots (two per lane) are loaded together.
    constexpr int RPL = (FCAPH + 63) / 64;
    auto for_records = [&](auto&& f) {
#pragma unroll 1
      for (int st = 0; st < FNW; ++st) {
        const int n = __builtin_amdgcn_readlane((int)nrec, st);
        const uint32_t* src = &sm.u.s.cand[u][hf][st][0][0];
        uint2 rc[RPL];
#pragma unroll
        for (int it = 0; it < RPL; ++it) {
          const int i = it * 64 + lane;
          rc[it] = i < n ? *reinterpret_cast<const uint2*>(src + 2 * i) : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int it = 0; it < RPL; ++it)
          if (it * 64 < n) f(it * 64 + lane < n, (rc[it].y >> 16) & 1u, rc[it].x, rc[it].y & 0xFFFFu);   // uniform
      }
    };
    // bm[E][u] as 32-bit words: word 2 (E FU + u) + (g >> 1), bits 16 (g & 1) + (e & 15)
    auto select = [&](int j, uint32_t e) {
      atomicOr(&bm32[(((e >> 4) * FU + u) << 1) + hf], 1u << ((j << 4) + (e & 15u)));
    };
    // token slot j's half of the scratch row: 128 bins (padded) or a 64-pair list
    auto hrow = [&](int j) { return sm.scr[wave] + j * (SROW / 2); };
    int tt[2], ne[2];
    bool act[2], fbk[2];
    uint32_t need[2], lo[2], sh[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      tt[j] = unit_token<HI>(u, g0 + j);
      ne[j] = tt[j] < nt ? row_len(a, b, t0 + tt[j]) : 0;
      act[j] = ne[j] > k;
      fbk[j] = false;
      uint32_t nab = 0;
      if (act[j]) {
        const int nE = (ne[j] + 15) >> 4;
        for (int E = lane; E < nE; E += 64) nab += (uint32_t)__popc(bm16[(E * FU + u) * 4 + g0 + j]);
        nab = wave_sum_u32(nab);
        if (sovf || nab > (uint32_t)k) { fbk[j] = true; act[j] = false; }
        else if (nab == (uint32_t)k) act[j] = false;         // the entries above the band are the k
      }
      need[j] = (uint32_t)k - nab;
      const uint32_t lk = act[j] ? sm.lo_key[tt[j]] : 0u, hk = act[j] ? sm.hi_key[tt[j]] : 0u;
      const uint32_t span = hk > lk ? hk - lk : 1u;
      lo[j] = lk;
      sh[j] = span <= 128u ? 0u : (uint32_t)(32 - __clz((int)(span - 1u))) - 7u;
    }
    if (act[0] || act[1]) {                                  // uniform
      // histograms of both tokens' records over their band ranges
      for (int i = lane; i < SROW; i += 64) sm.scr[wave][i] = 0u;
      wave_sync();
      uint32_t nc0 = 0, nc1 = 0;
      for_records([&](bool ok, uint32_t j, uint32_t key, uint32_t) {
        if (ok && (j ? act[1] : act[0])) {
          atomicAdd(&hrow((int)j)[spad((int)((key - (j ? lo[1] : lo[0])) >> (j ? sh[1] : sh[0])))], 1u);
          if (j) ++nc1; else ++nc0;
        }
      });
      const uint32_t nc[2] = {wave_sum_u32(nc0), wave_sum_u32(nc1)};
      wave_sync();
      uint32_t bb[2] = {0u, 0u}, rem[2] = {0u, 0u}, n1[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!act[j]) continue;
        if (need[j] > nc[j]) { fbk[j] = true; act[j] = false; continue; }   // the band holds too few
        uint32_t ab;
        wave_find_bin(128, need[j], [&](int i) { return hrow(j)[spad(i)]; }, bb[j], ab);
        rem[j] = need[j] - ab;                               // >= 1 still needed from bin bb
        n1[j] = hrow(j)[spad((int)bb[j])];
      }
      wave_sync();
      // records above the boundary bin are selected; those in it are gathered
      // (when at most 64) as (key, entry) pairs into the token's half row
      uint32_t at0 = 0, at1 = 0;
      for_records([&](bool ok, uint32_t j, uint32_t key, uint32_t e) {
        const bool on = ok && (j ? act[1] : act[0]);
        const uint32_t bin = (key - (j ? lo[1] : lo[0])) >> (j ? sh[1] : sh[0]);
        const uint32_t bj = j ? bb[1] : bb[0];
        if (on && bin > bj) select((int)j, e);
        const bool gat = on && bin == bj && (j ? n1[1] : n1[0]) <= 64u;
        const uint64_t m0 = __ballot(gat && j == 0u), m1 = __ballot(gat && j == 1u);
        if (gat) {
          const uint32_t slot = j ? at1 + lanes_below(m1) : at0 + lanes_below(m0);
          hrow((int)j)[2 * slot] = key;
          hrow((int)j)[2 * slot + 1] = e;
        }
        at0 += (uint32_t)__popcll(m0);
        at1 += (uint32_t)__popcll(m1);
      });
      wave_sync();
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (!act[j]) continue;
        uint32_t* row = hrow(j);
        uint32_t cnt1 = n1[j], rm = rem[j];
        uint32_t lo2 = lo[j] + (bb[j] << sh[j]), sh2 = sh[j];   // the boundary bin's key range
        bool ties = false;
        // refine a crowded boundary bin over its own range until it holds at
        // most 64 records or a single key
#pragma unroll 1
        while (cnt1 > 64u) {
          if (sh2 == 0) { ties = true; break; }
          const uint32_t bspan = 1u << sh2, sh3 = sh2 > 7u ? sh2 - 7u : 0u;
          for (int i = lane; i < SROW / 2; i += 64) row[i] = 0u;
          wave_sync();
          for_records([&](bool ok, uint32_t jj, uint32_t key, uint32_t) {
            if (ok && jj == (uint32_t)j && key - lo2 < bspan) atomicAdd(&row[spad((int)((key - lo2) >> sh3))], 1u);
          });
          wave_sync();
          uint32_t b3, ab3;
          wave_find_bin(128, rm, [&](int i) { return row[spad(i)]; }, b3, ab3);
          rm -= ab3;
          cnt1 = row[spad((int)b3)];
          wave_sync();
          uint32_t at = 0;
          for_records([&](bool ok, uint32_t jj, uint32_t key, uint32_t e) {
            const bool in = ok && jj == (uint32_t)j && key - lo2 < bspan;
            const uint32_t bin = (key - lo2) >> sh3;
            if (in && bin > b3) select(j, e);
            const bool gat = in && bin == b3 && cnt1 <= 64u;
            const uint64_t m = __ballot(gat);
            if (gat) {
              const uint32_t slot = at + lanes_below(m);
              row[2 * slot] = key;
              row[2 * slot + 1] = e;
            }
            at += (uint32_t)__popcll(m);
          });
          wave_sync();
          lo2 += b3 << sh3;
          sh2 = sh3;
        }
        if (!ties) {
          // rank of each gathered record among them: larger key first, then lower index
          const uint32_t kl = lane < (int)cnt1 ? row[2 * lane] : 0u;
          const uint32_t el = lane < (int)cnt1 ? row[2 * lane + 1] : 0u;
          uint32_t rank = 0;
          for (uint32_t q = 0; q < cnt1; ++q) {
            const uint32_t kq = (uint32_t)__builtin_amdgcn_readlane((int)kl, (int)q);
            const uint32_t eq = (uint32_t)__builtin_amdgcn_readlane((int)el, (int)q);
            rank += (kq > kl || (kq == kl && eq < el)) ? 1u : 0u;
          }
          if (lane < (int)cnt1 && rank < rm) select(j, el);
        } else {
          // more than 64 records share the key lo2: the rm of lowest index, one
          // 4096-entry range at a time through a bitmap in the half row
#pragma unroll 1
          for (int e0 = 0; e0 < ne[j] && rm > 0u; e0 += 4096) {
            for (int i = lane; i < SROW / 2; i += 64) row[i] = 0u;
            wave_sync();
            for_records([&](bool ok, uint32_t jj, uint32_t key, uint32_t e) {
              if (ok && jj == (uint32_t)j && key == lo2 && e - (uint32_t)e0 < 4096u)
                atomicOr(&row[(e - (uint32_t)e0) >> 5], 1u << (e & 31u));
            });
            wave_sync();
            uint32_t wv[2], c = 0;
#pragma unroll
            for (int q = 0; q < 2; ++q) { wv[q] = row[2 * lane + q]; c += (uint32_t)__popc(wv[q]); }
            const uint32_t incl = wave_incl_scan(c);
            uint32_t pos = incl - c;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              uint32_t w = wv[q];
              while (w && pos < rm) {
                const int bit = __ffs(w) - 1;
                w &= w - 1;
                select(j, (uint32_t)(e0 + (2 * lane + q) * 32 + bit));
                ++pos;
              }
            }
            const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
            rm -= min(tot, rm);
            wave_sync();
          }
        }
        wave_sync();
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (tt[j] >= nt) continue;                             // uniform
      int32_t* idx = a.idx_out + ((size_t)b * a.Tq + t0 + tt[j]) * k;
      if (ne[j] <= k) {
        for (int i = lane; i < k; i += 64) idx[i] = i < ne[j] ? i : -1;
        continue;
      }
      if (fbk[j]) {
        if (lane == 0) { sm.fb[tt[j]] = 1u; count_event(CNT_PREFILL_FALLBACK); }
        continue;                                            // written by the exact select below
      }
      // the token's bitmap fields, group E = E0 + lane, in ascending order
      const int nE = (ne[j] + 15) >> 4;
      uint32_t base = 0;
      for (int E0 = 0; E0 < nE; E0 += 64) {
        const int E = E0 + lane;
        uint32_t w = E < nE ? (uint32_t)bm16[(E * FU + u) * 4 + g0 + j] : 0u;
        const uint32_t c = (uint32_t)__popc(w);
        const uint32_t incl = wave_incl_scan(c);
        uint32_t pos = base + incl - c;
        while (w) {
          const int bit = __ffs(w) - 1;
          w &= w - 1;
          if (pos < (uint32_t)k) idx[pos] = E * 16 + bit;
          ++pos;
        }
        base += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      }
      for (uint32_t i = base + lane; i < (uint32_t)k; i += 64) idx[i] = -1;
    }
  }
  __syncthreads();
  // ---- exact fallback for tokens whose band missed or overflowed ----
  bool any_fb = false;
  for (int tt = 0; tt < nt; ++tt) any_fb |= sm.fb[tt] != 0u;
  if (any_fb) load_operands();                               // uniform
  for (int tt = 0; tt < nt; ++tt) {
    if (!sm.fb[tt]) continue;                                // uniform: LDS after a barrier
    const int ne = row_len(a, b, t0 + tt);
    float* srow = reinterpret_cast<float*>(a.ws) + ((size_t)b * a.Tq + t0 + tt) * nc_pad(a.Nc_cap);
    pass(0, FSTEP, [&](int u, int e, float sc, bool valid, int) {
      if (valid && tok[u] == tt) srow[e] = sc;
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

hipError_t counters_device_ptr(unsigned long long** p) {
  static std::mutex mu;
  static std::map<int, unsigned long long*> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(g_counters));
    if (e != hipSuccess) return e;
    it = cache.emplace(dev, reinterpret_cast<unsigned long long*>(q)).first;
  }
  *p = it->second;
  return hipSuccess;
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

bool indexer_long_path(const IndexerArgs& a) {
  return a.B > 0 && a.Tq > 0 && !use_fused_prefill(a) && use_long_path(a.Tq, a.Nc_cap);
}

hipError_t launch_indexer_scores(const IndexerArgs& a, hipStream_t st) {
  if (!indexer_long_path(a)) return hipErrorInvalidValue;
  switch (a.qk) {
    case QK_F32: launch_scores_di<QK_F32>(a, st, true); break;
    case QK_BF16: launch_scores_di<QK_BF16>(a, st, true); break;
    case QK_FP8: launch_scores_di<QK_FP8>(a, st, true); break;
    case QK_FP4: launch_scores_di<QK_FP4>(a, st, true); break;
  }
  return hipGetLastError();
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
  if (lp) hipLaunchKernelGGL(long_pick_kernel, dim3(a.B * a.Tq), dim3(1024), 0, st, a);
  else hipLaunchKernelGGL(topk_row_kernel, dim3(a.Tq, a.B), dim3(TOPK_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
