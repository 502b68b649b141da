// Lightning indexer scores + top-k selection.
// Method: DeepSeek-V4 summary (hyper.ai), "Method", CSA paragraph — a
// lightning indexer selects the top-k compressed entries; aiboss88 "Technical
// Principles", CSA bullet (index scores, top-k sparse selection) and FP4 bullet
// (FP4 indexer QK path, FP8 for the extra dynamic range).  Form implemented:
//   I[t,j] = sum_h w[t,h] * max(0, qI[t,h] . KIc_j),   j < floor((t+1)/m)
// then the k largest I[t,.] with equal scores going to the lower j, emitted
// ascending by j and padded with -1.
//
// Score kernel: the (token, head) rows of qI form the MFMA A operand (16 rows
// = 16/HI tokens), compressed indexer keys form B (16 entries per MFMA), so the
// 16x16 accumulator hands every lane the HI head dots of one token for one
// entry: ReLU and the head weighting happen in-lane.  FP8/FP4 codes are widened
// exactly to bf16 in registers (E4M3 and E2M1 x E8M0 values are all bf16
// values); products are exact and accumulate in fp32.
//
// Top-k kernel: one workgroup per query row.  The scores are non-negative
// (+0 for ReLU'd zeros), so their fp32 bit patterns order like the values and
// an 11/11/10-bit radix select finds the k-th largest key tau and how many
// entries equal to tau are needed; a chunked, index-ordered compaction then
// takes every key > tau and the lowest-indexed keys == tau, which yields the
// ascending index list directly.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

static constexpr int SCORE_WG_ENTRIES = 256;   // 4 waves x 4 tiles x 16 entries

__host__ __device__ __forceinline__ int nc_pad(int Nc_cap) { return (Nc_cap + 63) & ~63; }

// ---------------- operand loaders: 8 k-values -> one fragment --------------
// qk element encodings
template <int QK> struct QkTraits;
template <> struct QkTraits<QK_F32> { using Elem = float; using F = Frag<float>; };
template <> struct QkTraits<QK_BF16> { using Elem = bf16; using F = Frag<bf16>; };
template <> struct QkTraits<QK_FP8> { using Elem = uint8_t; using F = Frag<bf16>; };
template <> struct QkTraits<QK_FP4> { using Elem = uint8_t; using F = Frag<bf16>; };

// E4M3 code -> bf16 bits (exact).
__device__ __forceinline__ uint32_t e4m3_to_bf16_bits(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8;
  const uint32_t em = c & 0x7Fu;
  const uint32_t e = em >> 3;
  // normal: exponent e-7 -> bf16 exponent e+120; mantissa 3 bits -> top of 7
  const uint32_t nrm = (em << 4) + (120u << 7);
  // subnormal: (c & 7) * 2^-9, exact in fp32
  const uint32_t sub = __float_as_uint((float)(em & 7u) * 0.001953125f) >> 16;
  return s | (e ? nrm : sub);
}
// E2M1 code (low 4 bits) times 2^(E-127) -> fp32 (exact).
__device__ __forceinline__ float e2m1_val(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, f = c & 1u;
  float mag = e ? (1.f + 0.5f * (float)f) * (float)(1u << e) * 0.5f : 0.5f * (float)f;
  return (c & 8u) ? -mag : mag;
}

// Load the fragment for a row of `dI` k-values: elements k0 .. k0+7.
// FP8: `row` points at the codes of the row (scale applied by the caller).
// FP4: `row` points at packed codes; `sc` at the row's E8M0 scales.
template <int QK>
__device__ __forceinline__ void load_qk_frag(typename QkTraits<QK>::F& f, const void* row,
                                             const uint8_t* sc, int k0) {
  if constexpr (QK == QK_F32) {
    frag_load(f, reinterpret_cast<const float*>(row) + k0);
  } else if constexpr (QK == QK_BF16) {
    frag_load(f, reinterpret_cast<const bf16*>(row) + k0);
  } else if constexpr (QK == QK_FP8) {
    const uint2 c = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(row) + k0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w = i ? c.y : c.x;
      f.v[2 * i] = e4m3_to_bf16_bits(w & 0xFF) | (e4m3_to_bf16_bits((w >> 8) & 0xFF) << 16);
      f.v[2 * i + 1] = e4m3_to_bf16_bits((w >> 16) & 0xFF) | (e4m3_to_bf16_bits(w >> 24) << 16);
    }
  } else {
    const uint32_t c = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(row) + k0 / 2);
    const float scl = __uint_as_float((uint32_t)sc[k0 / 32] << 23);   // 2^(E-127)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t byte = (c >> (8 * i)) & 0xFF;
      const uint32_t lo = __float_as_uint(e2m1_val(byte & 0xF) * scl) >> 16;
      const uint32_t hi = __float_as_uint(e2m1_val(byte >> 4) * scl) >> 16;
      f.v[i] = lo | (hi << 16);
    }
  }
}

template <int QK> __device__ __forceinline__ size_t qk_row_bytes(int dI) {
  if constexpr (QK == QK_F32) return (size_t)dI * 4;
  else if constexpr (QK == QK_BF16) return (size_t)dI * 2;
  else if constexpr (QK == QK_FP8) return (size_t)dI;
  else return (size_t)dI / 2;
}

// ---------------------------------- scores ---------------------------------
template <int QK, int DI, int HI>
__global__ __launch_bounds__(256) void score_kernel(IndexerArgs a) {
  constexpr int TT = 16 / HI;        // tokens per workgroup
  constexpr int KC = DI / 32;        // 32-wide k chunks
  using F = typename QkTraits<QK>::F;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * TT;
  const int e_wg = blockIdx.x * SCORE_WG_ENTRIES;
  const int pos_first = a.pos0[b] + t0;
  const int t_last = min(t0 + TT, a.Tq) - 1;
  const int ne_max = min((a.pos0[b] + t_last + 1) / a.m, a.Nc_cap);
  if (e_wg >= ne_max) return;
  (void)pos_first;

  // A operand: query rows (token, head)
  const int r = lane & 15, g = lane >> 4;
  const int tq = t0 + r / HI, hq = r % HI;
  F qa[KC];
  const uint8_t* qsc = nullptr;
  const size_t qrow = ((size_t)b * a.Tq + tq) * HI + hq;
  const char* qptr = reinterpret_cast<const char*>(a.qi) + qrow * qk_row_bytes<QK>(DI);
  if constexpr (QK == QK_FP4) qsc = reinterpret_cast<const uint8_t*>(a.qi_scale) + qrow * (DI / 32);
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (tq < a.Tq) load_qk_frag<QK>(qa[c], qptr, qsc, 32 * c + 8 * g);
    else frag_zero(qa[c]);
  }
  // per-lane output rows 4g..4g+3 -> (token, head) weights (FP8: x query scale)
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
    const int e = e0 + r;                      // B operand column / output column
    const bool ev = e < ne_max;
    const size_t krow = (size_t)b * a.Nc_cap + (ev ? e : 0);
    const char* kptr = reinterpret_cast<const char*>(a.kic) + krow * qk_row_bytes<QK>(DI);
    const uint8_t* ksc = nullptr;
    if constexpr (QK == QK_FP4) ksc = reinterpret_cast<const uint8_t*>(a.kic_scale) + krow * (DI / 32);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      F kb;
      load_qk_frag<QK>(kb, kptr, ksc, 32 * c + 8 * g);
      mma16(acc, qa[c], kb);
    }
    float cs = 1.f;
    if constexpr (QK == QK_FP8) cs = reinterpret_cast<const float*>(a.kic_scale)[krow];
    // acc[i] = dot of row 4g+i with entry e
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
        const int ne = min((a.pos0[b] + t + 1) / a.m, a.Nc_cap);
        if (e < ne) ws[((size_t)b * a.Tq + t) * ldo + e] = s[u] * cs + 0.f;
      }
    }
  }
}

// ---------------------------------- top-k ----------------------------------
static constexpr int TOPK_NT = 512;
static constexpr int TOPK_LDS_KEYS = 12288;

struct TopkSmem {
  uint32_t hist[2048];
  uint32_t scan[TOPK_NT / 64];
  uint32_t bin, above;
};

// Locate, scanning from the top bin down, the bin where the running count
// first reaches `need`; writes the bin and the count strictly above it.
__device__ void find_bin(TopkSmem& sm, int nbins, uint32_t need) {
  const int per = nbins / TOPK_NT;              // 4 or 2 bins per thread
  const int tid = threadIdx.x;
  const int hi = nbins - tid * per;             // my bins: [hi-per, hi), scanned top-down
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += sm.hist[hi - 1 - i];
  uint32_t tot;
  const uint32_t excl = block_excl_scan<TOPK_NT>(local, sm.scan, &tot);
  if (excl < need && excl + local >= need) {
    uint32_t cum = excl;
    for (int i = 0; i < per; ++i) {
      const uint32_t h = sm.hist[hi - 1 - i];
      if (cum + h >= need) { sm.bin = hi - 1 - i; sm.above = cum; break; }
      cum += h;
    }
  }
  __syncthreads();
}

template <bool LDS_ROW>
__device__ void select_row(TopkSmem& sm, const uint32_t* __restrict__ row, int n, int k,
                           int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  if (tid == 0) { sm.bin = 0; sm.above = 0; }
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const int sh = p == 0 ? 21 : (p == 1 ? 10 : 0);
    const int nb = p == 2 ? 1024 : 2048;
    for (int i = tid; i < nb; i += TOPK_NT) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += TOPK_NT) {
      const uint32_t key = row[i];
      if ((key & pmask) == prefix) atomicAdd(&sm.hist[(key >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_bin(sm, nb, need);
    prefix |= sm.bin << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    need -= sm.above;
    __syncthreads();
  }
  const uint32_t tau = prefix, need_eq = need;

  uint32_t base = 0, eq_seen = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < n; c0 += TOPK_NT) {
    const int i = c0 + tid;
    const uint32_t key = i < n ? row[i] : 0u;
    const uint32_t is_gt = (i < n && key > tau) ? 1u : 0u;
    const uint32_t is_eq = (i < n && key == tau) ? 1u : 0u;
    uint32_t tot_eq;
    const uint32_t eq_x = block_excl_scan<TOPK_NT>(is_eq, sm.scan, &tot_eq);
    const uint32_t take = is_gt | ((is_eq && eq_seen + eq_x < need_eq) ? 1u : 0u);
    uint32_t tot_take;
    const uint32_t pos = block_excl_scan<TOPK_NT>(take, sm.scan, &tot_take);
    if (take && base + pos < (uint32_t)k) {
      idx_out[base + pos] = i;
      if (score_out) score_out[base + pos] = __uint_as_float(key);
    }
    base += tot_take;
    eq_seen += tot_eq;
    if (base >= (uint32_t)k) break;
  }
}

__global__ __launch_bounds__(TOPK_NT) void topk_kernel(IndexerArgs a) {
  __shared__ TopkSmem sm;
  __shared__ uint32_t rowbuf[TOPK_LDS_KEYS];
  const int t = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = max(0, min((a.pos0[b] + t + 1) / a.m, a.Nc_cap));
  const size_t orow = ((size_t)b * a.Tq + t) * a.topk;
  int32_t* idx = a.idx_out + orow;
  float* sco = a.score_out ? a.score_out + orow : nullptr;
  const uint32_t* src =
      reinterpret_cast<const uint32_t*>(a.ws) + ((size_t)b * a.Tq + t) * nc_pad(a.Nc_cap);
  if (n <= a.topk) {
    for (int i = tid; i < a.topk; i += TOPK_NT) {
      idx[i] = i < n ? i : -1;
      if (sco) sco[i] = i < n ? __uint_as_float(src[i]) : -INFINITY;
    }
    return;
  }
  if (n <= TOPK_LDS_KEYS) {
    for (int i = tid; i < n; i += TOPK_NT) rowbuf[i] = src[i];
    __syncthreads();
    select_row<true>(sm, rowbuf, n, a.topk, idx, sco);
  } else {
    select_row<false>(sm, src, n, a.topk, idx, sco);
  }
}

// --------------------------------- launch ----------------------------------
size_t indexer_workspace(int B, int Tq, int Nc_cap, int HI, int dI, int topk, int qk) {
  (void)HI; (void)dI; (void)topk; (void)qk;
  return (size_t)B * Tq * nc_pad(Nc_cap) * sizeof(float);
}

template <int QK, int DI, int HI>
static void launch_scores(const IndexerArgs& a, hipStream_t st) {
  const int TT = 16 / HI;
  const int ne_ub = std::min((a.max_pos + 1) / a.m, a.Nc_cap);
  dim3 grid((ne_ub + SCORE_WG_ENTRIES - 1) / SCORE_WG_ENTRIES, (a.Tq + TT - 1) / TT, a.B);
  if (grid.x == 0) return;
  hipLaunchKernelGGL((score_kernel<QK, DI, HI>), grid, dim3(256), 0, st, a);
}

template <int QK, int DI>
static void launch_scores_hi(const IndexerArgs& a, hipStream_t st) {
  if (a.HI == 1) launch_scores<QK, DI, 1>(a, st);
  else if (a.HI == 2) launch_scores<QK, DI, 2>(a, st);
  else launch_scores<QK, DI, 4>(a, st);
}

template <int QK>
static void launch_scores_di(const IndexerArgs& a, hipStream_t st) {
  if (a.dI == 32) launch_scores_hi<QK, 32>(a, st);
  else launch_scores_hi<QK, 64>(a, st);
}

hipError_t launch_indexer_topk(const IndexerArgs& a, hipStream_t st) {
  if (a.B == 0 || a.Tq == 0) return hipSuccess;
  switch (a.qk) {
    case QK_F32: launch_scores_di<QK_F32>(a, st); break;
    case QK_BF16: launch_scores_di<QK_BF16>(a, st); break;
    case QK_FP8: launch_scores_di<QK_FP8>(a, st); break;
    case QK_FP4: launch_scores_di<QK_FP4>(a, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3(a.Tq, a.B), dim3(TOPK_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
