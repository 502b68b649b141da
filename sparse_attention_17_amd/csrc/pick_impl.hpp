// Top-k selection pieces shared by the indexer kernels and the fused decode
// step: the long-row workspace layout (per-chunk candidates), the exact
// single-workgroup select, and the per-row pick over the chunks' candidates.
// Method: DeepSeek-V4 summary (hyper.ai), "Method", CSA paragraph — the
// lightning indexer keeps the top-k compressed entries; aiboss88 "Technical
// Principles", CSA bullet (top-k sparse selection).  Selected set: the k
// largest scores, equal scores going to the lower entry index, emitted
// ascending by index and padded with -1.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace csa {

// Increments event counter `which` of the array at `c` (if not NULL).
__device__ __forceinline__ void count_event_at(unsigned long long* c, int which) {
  if (c) atomicAdd(&c[which], 1ull);
}

// Index-list entries are stored with device scope (sc1: written through to the
// level coherent across the XCDs), so that attention workgroups of the same
// launch can read them (the fused decode step).
__device__ __forceinline__ void store_idx(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// decode score kernels: entries per chunk (one chunk per workgroup; 1024
// gives two rounds of resident workgroups on a 1M-entry batch, so one round's
// chunk cuts overlap the other's loads)
static constexpr int SCORE_CHUNK = 1024;
static constexpr int H1_BITS = 12;             // first radix digit (key bits 20..31)
static constexpr int H1_BINS = 1 << H1_BITS;
static constexpr int TOPK_NT = 512;
static constexpr int TOPK_LDS_KEYS = 12288;

__host__ __device__ __forceinline__ int nc_pad(int Nc_cap) { return (Nc_cap + 63) & ~63; }

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
      store_idx(idx_out + base + pos, i);
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
    store_idx(idx + i, i < n ? i : -1);
    if (sco) sco[i] = i < n ? __uint_as_float(src[i]) : -INFINITY;
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
static constexpr int PICK_BINS = 4096;         // 12-bit radix digits

// Sizes per workgroup shape: a 1024-thread pick (its own launch) handles rows
// of up to 4096 chunks with up to 30 slots per thread; a 256-thread pick
// (inside the fused decode-step kernel, LDS shared with attention) up to 512
// chunks with up to 64 slots per thread.
template <int NT> struct PickGeom;
template <> struct PickGeom<1024> {
  static constexpr int MAXCH = 4096, MAXPER = 30, STASH = 16384;
};
template <> struct PickGeom<256> {
  static constexpr int MAXCH = 512, MAXPER = 64, STASH = 8192;
};

template <int NT>
struct PickSmem {
  using G = PickGeom<NT>;
  static constexpr int WORDS = G::MAXPER * NT / 32;
  uint32_t hist[2][PICK_BINS];                 // alternating digit histograms
  uint32_t ccnt[G::MAXCH];                     // kept count per chunk (clamped to cap)
  uint32_t ccut[G::MAXCH];                     // cut key prefix per chunk
  uint32_t bm_gt[WORDS];                       // output bitmaps over slots
  uint32_t bm_eq[WORDS];
  uint32_t sel[G::STASH];                      // entry index of selected slots
  uint32_t wv[4][NT / 64];                     // per-wave partials
  uint32_t res[3];                             // bin, count above it, count in it
  uint32_t tau;                                // the first round's threshold (second round)
};
static_assert(sizeof(TopkSmem<1024>) <= sizeof(PickSmem<1024>), "fallback select aliases PickSmem");
static_assert(sizeof(TopkSmem<256>) <= sizeof(PickSmem<256>), "fallback select aliases PickSmem");

// Sum of the per-wave totals w[0 .. wave-1] (wave = this thread's wave):
// lane i < NT/64 reads w[i] once and a masked wave sum replaces a serial
// walk over the totals.
__device__ __forceinline__ uint32_t waves_below(const uint32_t* w, int wave) {
  const int lane = threadIdx.x & 63;
  return wave_sum_u32(lane < wave ? w[lane] : 0u);           // wave < 16
}

struct PickRow {
  int row, n, k, nch, cap, lg, nslot;
  int single;                                  // >= 0: one chunk of `single` uncut slots, no meta
  const uint2* meta;
  const uint2* cand;
  const uint32_t* src;
  int32_t* idx;
  float* sco;
  unsigned long long* counters;                // event counters (may be NULL)
};

// Outcome of one pick round.
enum PickStatus { PICK_DONE = 0, PICK_ROUND2 = 1, PICK_EXACT = 2 };

// Select for one row whose nslot fits PER slots per thread.  Slot s holds
// (key, entry) of the (s mod cap)-th kept entry of chunk s / cap; thread tid
// holds slots q * NT + tid (coalesced loads).  Every loop runs exactly
// PER times, and the output bitmaps are built from wave ballots.  Returns
// PICK_DONE with the index list written; PICK_ROUND2 when some chunk may have
// dropped (or could not keep) an entry above the candidates' k-th largest
// key, which is then left in sm.tau (a lower bound of the row's k-th largest
// key, as the candidates are a subset of the row); PICK_EXACT when the
// candidates number fewer than k.
template <int NT, int PER>
__device__ __forceinline__ int pick_body(PickSmem<NT>& sm, const PickRow& R) {
  using G = PickGeom<NT>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr uint2 EMPTY = {0u, 0xFFFFFFFFu};
  const int k = R.k, cap = R.cap, lg = R.lg, nslot = R.nslot, nch = R.nch;

  // ---- 1. candidate slots and chunk records, requested together ----
  uint2 kv[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) kv[q] = R.cand[min(q * NT + tid, nslot - 1)];
  uint32_t part = 0;
  int ovf = 0;
  for (int c = tid; c < nch; c += NT) {
    const uint2 r = R.single >= 0 ? uint2{(uint32_t)R.single, CUT_ALL} : R.meta[c];
    sm.ccnt[c] = min(r.x, (uint32_t)cap);
    sm.ccut[c] = r.y;
    ovf |= r.x > (uint32_t)cap;
    part += min(r.x, (uint32_t)cap);
  }
  for (int i = tid; i < PICK_BINS; i += NT) sm.hist[0][i] = 0;
  __syncthreads();

  // ---- 2. mask empty slots; candidate total, key range, overflow ----
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int s = q * NT + tid;
    const bool ok = s < nslot && (s & (cap - 1)) < (int)sm.ccnt[min(s >> lg, G::MAXCH - 1)];
    kv[q].x = ok ? kv[q].x : EMPTY.x;
    kv[q].y = ok ? kv[q].y : EMPTY.y;
    kmin = ok ? min(kmin, kv[q].x) : kmin;
    kmax = ok ? max(kmax, kv[q].x) : kmax;
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  part = wave_sum_u32(part);
  ovf = wave_max_u32((uint32_t)ovf) != 0u;
  if (lane == 0) { sm.wv[0][wave] = part; sm.wv[1][wave] = kmin; sm.wv[2][wave] = kmax; sm.wv[3][wave] = ovf; }
  __syncthreads();
  uint32_t total = 0;
  kmin = 0xFFFFFFFFu; kmax = 0;
  int overflow = 0;                                          // a chunk kept more than its slots
#pragma unroll
  for (int w = 0; w < (NT / 64); ++w) {
    total += sm.wv[0][w];
    kmin = min(kmin, sm.wv[1][w]);
    kmax = max(kmax, sm.wv[2][w]);
    overflow |= sm.wv[3][w];
  }
  const int bad = total < (uint32_t)k;                       // uniform

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
      const int nbs = max(nb, NT);                       // bins scanned
      uint32_t* hist = sm.hist[buf];
      for (int i = tid; i < PICK_BINS; i += NT) sm.hist[buf ^ 1][i] = 0;   // next pass's buffer
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const uint2 v = kv[q];
        if (v.y != EMPTY.y && (v.x & pmask) == prefix) atomicAdd(&hist[(v.x >> sh) & (nb - 1)], 1u);
      }
      __syncthreads();
      // top-down scan: thread tid owns bins [nbs - pb*(tid+1), nbs - pb*tid)
      const int pb = nbs / NT;
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
  int unsafe = bad | overflow;
  if (!bad)
    for (int c = tid; c < nch; c += NT) {
      const uint32_t cut = sm.ccut[c];
      unsafe |= cut != CUT_ALL && tau < (cut << 12);
    }
  // slot bitmaps of keys > tau and keys == tau, one ballot per 64 slots (each
  // word has one writer: no atomics, no clearing); selected entries kept
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const uint2 v = kv[q];
    const int s = q * NT + tid;
    const bool valid = v.y != EMPTY.y;
    const bool gt = valid && v.x > tau, eq = valid && v.x == tau;
    if ((gt || eq) && s < G::STASH) sm.sel[s] = v.y;
    const uint64_t bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      const int w0 = (q * NT + wave * 64) >> 5;
      sm.bm_gt[w0] = (uint32_t)bg;
      sm.bm_gt[w0 + 1] = (uint32_t)(bg >> 32);
      sm.bm_eq[w0] = (uint32_t)be;
      sm.bm_eq[w0 + 1] = (uint32_t)(be >> 32);
    }
  }
  if (__syncthreads_or(unsafe)) {
    if (tid == 0) sm.tau = tau;
    __syncthreads();
    return bad ? PICK_EXACT : PICK_ROUND2;
  }

  // ---- 4. output in slot order (= ascending entry order): the bitmap words
  // are split into Q parts of L slots; thread tid owns UPT consecutive parts
  // starting at part tid * UPT (so the threads hold the slots in order): keys
  // > tau, and the first `need` keys == tau over the whole row ----
  constexpr int NWORDS = PER * NT / 32;
  constexpr int Q = NT / NWORDS >= 4 ? 4 : NT / NWORDS >= 2 ? 2 : 1;
  constexpr int L = 32 / Q;
  constexpr int UPT = (NWORDS * Q + NT - 1) / NT;             // 1 unless NWORDS > NT
  constexpr uint32_t LMASK = L == 32 ? 0xFFFFFFFFu : (1u << L) - 1u;
  uint32_t wgt[UPT], weq[UPT];
  uint32_t pgt = 0, peq = 0;
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int unit = tid * UPT + u, word = unit / Q, wpart = unit % Q;
    wgt[u] = word < NWORDS ? (sm.bm_gt[word] >> (wpart * L)) & LMASK : 0u;
    weq[u] = word < NWORDS ? (sm.bm_eq[word] >> (wpart * L)) & LMASK : 0u;
    pgt += (uint32_t)__popc(wgt[u]);
    peq += (uint32_t)__popc(weq[u]);
  }
  const uint32_t inc_gt = wave_incl_scan(pgt), inc_eq = wave_incl_scan(peq);
  if (lane == 63) { sm.wv[1][wave] = inc_gt; sm.wv[2][wave] = inc_eq; }
  __syncthreads();
  uint32_t gt_before = inc_gt - pgt, eq_before = inc_eq - peq;
  gt_before += waves_below(sm.wv[1], wave);
  eq_before += waves_below(sm.wv[2], wave);
  uint32_t pos = gt_before + min(eq_before, need);
  uint32_t e_seen = eq_before;
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    uint32_t take = wgt[u];
    for (uint32_t m = weq[u]; m; m &= m - 1) {
      const int bit = __ffs(m) - 1;
      if (e_seen++ < need) take |= 1u << bit;
    }
    const int unit = tid * UPT + u;
    const int s0 = (unit / Q) * 32 + (unit % Q) * L;
    for (; take; take &= take - 1) {
      const int s = s0 + __ffs(take) - 1;
      if (pos < (uint32_t)k) {
        store_idx(R.idx + pos, (int32_t)(s < G::STASH ? sm.sel[s] : R.cand[s].y));
        if (R.sco) R.sco[pos] = __uint_as_float(R.cand[s].x);
      }
      ++pos;
    }
  }
  return PICK_DONE;
}

// pick_body with the slots-per-thread body chosen for R.nslot (a uniform
// branch); rows needing more than the largest body take PICK_EXACT.
template <int NT>
__device__ __forceinline__ int pick_round(PickSmem<NT>& sm, const PickRow& R) {
  using G = PickGeom<NT>;
  const int per = (R.nslot + NT - 1) / NT;
  if (per > G::MAXPER || R.nch > G::MAXCH) return PICK_EXACT;
  if (per <= 8) return pick_body<NT, 8>(sm, R);
  if (per <= 16) return pick_body<NT, 16>(sm, R);
  if (G::MAXPER <= 32 || per <= 32) return pick_body<NT, (G::MAXPER < 32 ? G::MAXPER : 32)>(sm, R);
  return pick_body<NT, G::MAXPER>(sm, R);
}

// Second round for a row whose chunk cuts may have dropped an entry above the
// first round's threshold tau (a lower bound of the row's k-th largest key):
// chunk by chunk, in entry order, the entries with key >= tau — a safe chunk's
// kept candidates, every stored score of an unsafe or overflowed chunk — are
// compacted into the row's free candidate slots (after the first round's),
// where one uncut chunk of them is picked exactly.  Returns PICK_EXACT when
// they do not fit.
template <int NT>
__device__ __forceinline__ int pick_second_round(PickSmem<NT>& sm, const PickRow& R) {
  using G = PickGeom<NT>;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t tau = sm.tau;
  uint32_t* cnt = sm.hist[1];                                // per-chunk counts, then offsets
  auto chunk_kind = [&](int c) {                             // 0 safe, 1 rescan the stored scores
    const uint2 r = R.meta[c];
    return (r.y != CUT_ALL && tau < (r.y << 12)) || r.x > (uint32_t)R.cap ? 1 : 0;
  };
  // entries of chunk c that the second round keeps: each wave takes chunks
  // wave, wave + NW, ...; pass 0 counts, pass 1 writes at the chunk's offset
  uint2* out = const_cast<uint2*>(R.cand) + R.nslot;
  const int room = min(R.nch * SCORE_CHUNK - R.nslot, G::MAXPER * NT);
  for (int pass = 0; pass < 2; ++pass) {
    for (int c = wave; c < R.nch; c += NW) {
      const bool rescan = chunk_kind(c) != 0;                // wave-uniform
      const int len = rescan ? min(SCORE_CHUNK, R.n - c * SCORE_CHUNK) : (int)sm.ccnt[c];
      uint32_t pos = pass ? cnt[c] : 0u;
      for (int i0 = 0; i0 < len; i0 += 64) {
        const int i = i0 + lane;
        uint32_t key = 0, ent = 0;
        if (i < len) {
          if (rescan) { key = R.src[c * SCORE_CHUNK + i]; ent = (uint32_t)(c * SCORE_CHUNK + i); }
          else { const uint2 v = R.cand[c * R.cap + i]; key = v.x; ent = v.y; }
        }
        const bool keep = i < len && key >= tau;
        const uint64_t m = __ballot(keep);
        if (pass && keep) {
          const uint32_t at = pos + (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (at < (uint32_t)room) out[at] = uint2{key, ent};
        }
        pos += (uint32_t)__popcll(m);
      }
      if (!pass && lane == 0) cnt[c] = pos;
    }
    __syncthreads();
    if (!pass) {
      // exclusive scan of the chunk counts (chunks tid * per .. : in order)
      const int per = (R.nch + NT - 1) / NT;
      uint32_t local = 0;
      for (int j = 0; j < per; ++j) {
        const int c = tid * per + j;
        local += c < R.nch ? cnt[c] : 0u;
      }
      const uint32_t incl = wave_incl_scan(local);
      if (lane == 63) sm.wv[0][wave] = incl;
      __syncthreads();
      uint32_t run = incl - local + waves_below(sm.wv[0], wave);
      if (tid == NT - 1) sm.res[0] = run + local;              // total
      for (int j = 0; j < per; ++j) {
        const int c = tid * per + j;
        if (c < R.nch) { const uint32_t v = cnt[c]; cnt[c] = run; run += v; }
      }
      __syncthreads();
      if (sm.res[0] > (uint32_t)room) return PICK_EXACT;     // uniform
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int total = (int)sm.res[0];
  PickRow R2 = R;
  R2.nch = 1;
  R2.single = total;
  R2.cand = out;
  int cap2 = 32;
  while (cap2 < total) cap2 <<= 1;
  R2.cap = cap2;                                             // one chunk: slot s < total is entry s
  R2.lg = 31 - __clz(cap2);
  R2.nslot = total;                                          // loads stay inside the written slots
  return pick_round<NT>(sm, R2);
}

// One workgroup picks row `row`: the row's geometry, then the body
// specialised for its slots per thread (a uniform branch).  Rows needing more
// slots or chunks than the LDS holds take the exact select over the stored
// scores.
template <int NT>
__device__ __forceinline__ void pick_row(PickSmem<NT>& sm, const IndexerArgs& a, int row, unsigned long long* counters) {
  using G = PickGeom<NT>;
  PickRow R;
  R.row = row;
  R.counters = counters;
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
    write_all_eligible(R.n, R.k, R.src, R.idx, R.sco, NT);
    return;
  }
  R.nch = (R.n + SCORE_CHUNK - 1) / SCORE_CHUNK;
  R.cap = chunk_cap_n(R.k, R.n);
  R.lg = 31 - __clz(R.cap);                                  // cap is a power of two
  R.nslot = R.nch << R.lg;                                   // <= L.nch * SCORE_CHUNK
  R.single = -1;
  int st = pick_round<NT>(sm, R);
  if (st == PICK_ROUND2) {
    if (threadIdx.x == 0) count_event_at(counters, CNT_DECODE_SECOND_ROUND);
    st = pick_second_round<NT>(sm, R);
  }
  if (st != PICK_DONE) {
    if (threadIdx.x == 0) count_event_at(counters, CNT_DECODE_FALLBACK);
    select_row<NT>(*reinterpret_cast<TopkSmem<NT>*>(&sm.hist[0][0]), R.src, R.n, R.k, R.idx, R.sco);
  }
}

}  // namespace csa
