// Core attention kernels (templates) for CSA (selected compressed entries + sliding window + sink)
// and HCA (every completed m'-block + optional window + sink).
// Method: DeepSeek-V4 summary (hyper.ai), "Method": CSA core attention is MQA
// over the top-k compressed entries with shared keys and values; HCA attends
// densely over its heavily compressed entries; both add a sliding-window
// branch.  aiboss88 "Technical Principles", CSA bullet: sliding window plus an
// attention sink.  Form implemented (one softmax over all three parts):
//   o = sum_j e^(l_j - M) v_j / (e^(s_h - M) + sum_j e^(l_j - M)),
//   l_j = scale * q.k_j,  lse = M + ln(denominator).
//
// Mapping (MI355X, wave64, MFMA 32x32x16 bf16 / 32x32x2 fp32):
//   * a workgroup owns a tile of query rows = (token, head) pairs: all H
//     heads of one token for CSA (each token has its own key set), several
//     tokens x H heads for HCA (all share the block prefix);
//   * keys are staged KT=64 at a time in LDS: K row-major, V transposed;
//   * each wave computes S^T = K Q^T for its 32 query rows, so every lane owns
//     one query column: the online-softmax statistics stay in-lane (one
//     cross-half shuffle), the probabilities already sit in the B-operand
//     layout of O^T = V^T P^T, and the O^T accumulator rescale is per lane;
//   * decode (one query token) splits the key list over workgroups and a
//     combine kernel merges the partial (o, max, sum) in fixed split order,
//     so results do not depend on the batch size.
#pragma once
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>
#include <climits>
#include <type_traits>

namespace csa {

static constexpr int KT = 64;
static constexpr float LOG2E = 1.4426950408889634f;
static constexpr float LN2 = 0.6931471805599453f;

struct AttnGeom {
  int TT;          // tokens per tile
  int nsplit;      // key splits
  int kps;         // keys per split (multiple of KT)
  float scale_log2;
};

__host__ __device__ __forceinline__ int hca_ne(int pos, int mp, int cap) {
  return max(0, min((pos + 1) / mp, cap));
}

template <typename T>
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of the 4-key block kb (0..15) in row `dim` of the transposed V
// tile: blocks are XOR-swizzled by the row's 8-dim group so that the staging
// stores (one 4-key block for each of 8 consecutive dims per lane, lanes 8
// dims apart) spread over the LDS banks; the MFMA operand reads apply the same map.
__device__ __forceinline__ int vt_block(int dim, int kb) { return kb ^ ((dim >> 3) & 15); }

// RW row-waves (32 query rows each) x KG key groups (KG=2: each wave of a pair
// takes one 32-key half of every 64-key tile; the two partial softmax states
// are merged in LDS at the end).  PF key tiles are in flight ahead of the one
// being computed (PF=2 for split decode: a 128-key CSA split is then requested
// at once; FP8 caches keep one tile ahead).  Every instance fits 256 VGPRs,
// two waves per SIMD: two four-wave workgroups share a compute unit and one's
// loads overlap the other's math, or one eight-wave workgroup (256-row dense
// prefill tiles) holds it, its two halves staggered by the double-buffered
// key tiles.
// The body takes its workgroup's coordinates (token tile bx, split by,
// sequence bz) and the dynamic LDS block from the kernel that runs it.  COH
// (bit mask): COH_IDX reads the index row, COH_PART writes the split partials
// with device-scope (sc1) accesses, coherent across the XCDs' L2 caches, for
// an index producer or a merge running in the same launch.
static constexpr int COH_IDX = 1, COH_PART = 2;
__host__ __device__ constexpr bool attend_double_buffered(bool sparse, bool kv8, int rw, int pf) {
  return !sparse && !kv8 && rw == 8 && pf == 1;
}
template <typename T, int D, int RW, int KG, bool SPARSE, int PF, bool KV8 = false, bool VSH = false,
          int COH = 0>
__device__ __forceinline__ void attend_body(const AttendArgs& a, const AttnGeom& gm, int bx, int by,
                                            int bz, unsigned char* smem_raw) {
  static_assert(!KV8 || sizeof(T) == 2, "FP8 caches go with bf16 queries");
  constexpr int IDX_AUX = (COH & COH_IDX) ? 16 : 0;   // buffer-load cache policy: sc1 (device scope)
  static_assert(KV8 || !VSH, "a shared value entry is an FP8-cache layout");
  constexpr int NW = RW * KG;
  constexpr int NT = NW * 64;
  constexpr int NSUB = 2 / KG;                 // 32-key sub-tiles per wave per tile
  constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int KPAD = VEC;                    // Ks row padding (16 bytes)
  constexpr int VPAD = 4;                      // Vt row padding (elements)
  constexpr int KS = D + KPAD;                 // Ks row stride (elements)
  constexpr int VS = KT + VPAD;                // Vt row stride (elements)
  constexpr int DSTEP = D / 16;                // k-steps of S^T
  constexpr int DVT = D / 32;                  // 32-wide dv tiles of O^T
  static_assert(D <= 128, "the V-tile swizzle term (dim >> 3) must stay below 16");

  T* Ks = reinterpret_cast<T*>(smem_raw);
  T* Vt = Ks + KT * KS;
  // double-buffered key tiles (dense 256-row prefill tiles): the second
  // buffer starts DBUF elements after the first
  constexpr bool DB = attend_double_buffered(SPARSE, KV8, RW, PF);
  constexpr int DBUF = KT * KS + D * VS;
  // FP8 caches: the row scales of the tile's keys (1 for window rows), applied
  // to the logits of the code half and to the probabilities, in fp32
  float* kscl = reinterpret_cast<float*>(Vt + D * VS);
  float* vscl = kscl + KT;
  int* sel = KV8 ? reinterpret_cast<int*>(vscl + KT) : reinterpret_cast<int*>(Vt + D * VS);
  __shared__ uint32_t scan_sm[NW];
  __shared__ int s_nsel;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rw = wave % RW, kg = wave / RW;
  const int half = lane >> 5, col = lane & 31;
  const int b = bz, split = by;
  const int t0 = bx * gm.TT;
  const int tl = min(t0 + gm.TT, a.Tq) - 1;
  const int p0 = a.pos0[b];
  const int pos_first = p0 + t0, pos_last = p0 + tl;
  const int rp0 = a.raw_pos0 ? a.raw_pos0[b] : 0;

  // Buffer resources: a load outside a buffer's range returns zeros, so absent
  // keys, padding rows and masked slots are fetched without branches (which
  // also keeps every load of a tile in flight together).
  constexpr uint32_t OOB = 0x80000000u;                      // offset past every range
  constexpr uint32_t ROWB = D * sizeof(T);
  auto rsrc = [](const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
  };

  // ---- this wave's query fragments: loaded once into registers, issued
  // before anything else ----
  Frag<T> qfr[DSTEP];
  {
    const __amdgpu_buffer_rsrc_t rq =
        rsrc(reinterpret_cast<const T*>(a.q) + (size_t)b * a.Tq * a.H * D, (uint32_t)a.Tq * a.H * ROWB);
    const int r = rw * 32 + col;
    const int ttr = r / a.H, hr = r % a.H, tqr = t0 + ttr;
    const bool ok = ttr < gm.TT && tqr < a.Tq;
    const uint32_t base = (uint32_t)(tqr * a.H + hr) * ROWB + 8 * half * sizeof(T);
#pragma unroll
    for (int s = 0; s < DSTEP; ++s) {
      const uint32_t off = base + 16 * s * sizeof(T);
      if constexpr (sizeof(T) == 2) {
        qfr[s].v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, ok ? off : OOB, 0, 0));
      } else {
        const f32x4 lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, ok ? off : OOB, 0, 0));
        const f32x4 hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, ok ? off + 16 : OOB, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) { qfr[s].v[i] = lo[i]; qfr[s].v[4 + i] = hi[i]; }
      }
    }
  }

  // ---- the tile's key list: [compressed part][window part] ----
  const int kbeg = split * gm.kps;
  int ncomp, sel_base = 0;
  if constexpr (SPARSE) {
    const int32_t* ir = a.idx + ((size_t)b * a.Tq + t0) * a.topk;
    const __amdgpu_buffer_rsrc_t ri = rsrc(ir, (uint32_t)a.topk * 4);
    if (gm.nsplit > 1) {
      // split decode: this workgroup's own slots of the index row; slots whose
      // entry is invalid are masked out later
      ncomp = a.topk;
      sel_base = kbeg;
      const int ns = max(0, min(gm.kps, a.topk - kbeg));
      for (int i = tid; i < ns; i += NT)
        sel[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)(kbeg + i) * 4, 0, IDX_AUX);
      __syncthreads();
    } else {
      // one workgroup per token: compact the valid entries into LDS; each
      // thread owns a contiguous run of the index row, loaded in one round
      constexpr int RUN = (4096 + NT - 1) / NT;      // topk <= 4096
      const int i0 = tid * RUN;
      int ev[RUN];
      uint32_t cnt = 0;
#pragma unroll
      for (int q = 0; q < RUN; ++q) {
        const int i = i0 + q;
        const int v = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, i < a.topk ? (uint32_t)i * 4 : OOB, 0, IDX_AUX);
        ev[q] = i < a.topk ? v : -1;
      }
#pragma unroll
      for (int q = 0; q < RUN; ++q) cnt += (ev[q] >= 0 && ev[q] < a.Nc_cap) ? 1u : 0u;
      uint32_t base;
      uint32_t pos = block_excl_scan<NT>(cnt, scan_sm, &base);
#pragma unroll
      for (int q = 0; q < RUN; ++q)
        if (ev[q] >= 0 && ev[q] < a.Nc_cap) sel[pos++] = ev[q];
      if (tid == 0) s_nsel = (int)base;
      __syncthreads();
      ncomp = s_nsel;
    }
  } else {
    ncomp = hca_ne(pos_last, a.m_prime, a.Nc_cap);
  }
  const int wlo = a.window > 0 ? max(0, pos_first - a.window + 1) : 0;
  const int nwin = a.window > 0 ? pos_last - wlo + 1 : 0;
  const int nkeys = ncomp + nwin;
  const int kend = min(nkeys, kbeg + gm.kps);

  // ---- this lane's query row ----
  const int qr = rw * 32 + col;
  const int tt = qr / a.H, hq = qr % a.H;
  const int tq = t0 + tt;
  const bool qvalid = (tt < gm.TT) && (tq < a.Tq);
  const int qpos = p0 + tq;
  const int q_ne = SPARSE ? ncomp : hca_ne(qpos, a.m_prime, a.Nc_cap);
  const int q_wlo = max(0, qpos - a.window + 1);

  f32x16 o[DVT];
#pragma unroll
  for (int i = 0; i < DVT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const T* kcb = reinterpret_cast<const T*>(a.kc) + (size_t)b * a.Nc_cap * D;
  const T* vcb = reinterpret_cast<const T*>(a.vc) + (size_t)b * a.Nc_cap * D;
  const T* kwb = a.kw ? reinterpret_cast<const T*>(a.kw) + (size_t)b * a.R * D : nullptr;
  const T* vwb = a.vw ? reinterpret_cast<const T*>(a.vw) + (size_t)b * a.R * D : nullptr;
  // Facts that let whole tiles skip per-element masking (wave-uniform):
  // every window row is present in the raw buffer, and the smallest number of
  // compressed entries visible to any valid row of this wave.
  const bool win_ok = nwin == 0 || (kwb != nullptr && wlo - rp0 >= 0 && wlo + nwin - 1 - rp0 < a.R);
  int wave_min_ne = qvalid ? q_ne : INT_MAX;
  wave_min_ne = (int)wave_min_u32((uint32_t)wave_min_ne);                 // q_ne >= 0

  // byte offset of key slot s's row in the compressed / window buffers (OOB =
  // not there)
  const __amdgpu_buffer_rsrc_t rkc = rsrc(kcb, (uint32_t)a.Nc_cap * ROWB);
  const __amdgpu_buffer_rsrc_t rvc = rsrc(vcb, (uint32_t)a.Nc_cap * ROWB);
  const __amdgpu_buffer_rsrc_t rkw = rsrc(kwb, kwb ? (uint32_t)a.R * ROWB : 0u);
  const __amdgpu_buffer_rsrc_t rvw = rsrc(vwb, vwb ? (uint32_t)a.R * ROWB : 0u);
  // compressed entry held by key slot s, or -1
  auto ent = [&](int s) -> int {
    if (s < kbeg || s >= kend || s >= ncomp) return -1;
    const int e = SPARSE ? sel[s - sel_base] : s;
    return (e >= 0 && e < a.Nc_cap) ? e : -1;
  };
  auto comp_off = [&](int s) -> uint32_t {
    const int e = ent(s);
    return e >= 0 ? (uint32_t)e * ROWB : OOB;
  };
  // FP8 cache planes of this sequence
  constexpr int DN = D / 2;                                  // E4M3 dims of a K row (the rest is bf16)
  const size_t cb = (size_t)b * a.Nc_cap;
  const __amdgpu_buffer_rsrc_t rk8 = rsrc(KV8 ? (const uint8_t*)a.k8 + cb * DN : nullptr, KV8 ? (uint32_t)a.Nc_cap * DN : 0u);
  const __amdgpu_buffer_rsrc_t rkr = rsrc(KV8 ? (const uint16_t*)a.krope + cb * (D - DN) : nullptr,
                                          KV8 ? (uint32_t)a.Nc_cap * (D - DN) * 2 : 0u);
  constexpr bool vshared = VSH;                              // values = key rows (shared entry)
  const __amdgpu_buffer_rsrc_t rv8 = rsrc(KV8 && !vshared ? (const uint8_t*)a.v8 + cb * D : nullptr,
                                          KV8 && !vshared ? (uint32_t)a.Nc_cap * D : 0u);
  const __amdgpu_buffer_rsrc_t rks = rsrc(KV8 ? a.kscale + cb : nullptr, KV8 ? (uint32_t)a.Nc_cap * 4 : 0u);
  const __amdgpu_buffer_rsrc_t rvs = rsrc(KV8 && !vshared ? a.vscale + cb : nullptr,
                                          KV8 && !vshared ? (uint32_t)a.Nc_cap * 4 : 0u);
  // 8 codes of an FP8 row chunk (x, y), or zeros
  auto ld8 = [](const __amdgpu_buffer_rsrc_t& rc, int e, uint32_t off) -> u32x4 {
    const auto c = __builtin_amdgcn_raw_buffer_load_b64(rc, e >= 0 ? off : OOB, 0, 0);
    return u32x4{c[0], c[1], 0u, 0u};
  };
  // 8 E4M3 codes as 8 bf16 values: every E4M3 value is a bf16 value, so the
  // widening is exact; the row scale is applied later in fp32
  auto widen8 = [](const u32x4& r) -> u32x4 {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      o[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[w], 1.0f, false));
      o[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[w], 1.0f, true));
    }
    return o;
  };
  auto win_off = [&](int s) -> uint32_t {
    if (s < kbeg || s >= kend || s < ncomp) return OOB;
    const int r = wlo + (s - ncomp) - rp0;
    return (r >= 0 && r < a.R) ? (uint32_t)r * ROWB : OOB;
  };

  // ---- staging: all global loads of a tile are issued into registers first
  // (so they are in flight together), then written to LDS: K row-major, V
  // transposed.  Tiles that hold only compressed or only window keys read one
  // buffer; the tile that straddles both ORs the two (one of them is zero).
  constexpr int KCH = D / VEC;                               // 16-byte chunks per row
  constexpr int KLD = (KT * KCH + NT - 1) / NT;              // K chunks per thread
  constexpr int VTOT = (KT / 4) * KCH;                       // V tasks: 4 keys x 16 bytes
  constexpr int VTK = (VTOT + NT - 1) / NT;
  u32x4 kregA[KLD], vregA[VTK][4];
  u32x4 kregB[PF == 2 ? KLD : 1], vregB[PF == 2 ? VTK : 1][4];
  float sclA = 1.f, sclB = 1.f;                              // FP8 caches: one row scale per thread
  // K staging task c -> (row, 16-byte chunk): row-major for bf16 caches; for
  // FP8 caches chunk-major, so that a wave's 64 lanes share one chunk (and
  // with it the chunk's kind: codes or RoPE values)
  auto krow = [](int c) { return KV8 ? c % KT : c / KCH; };
  auto kch = [](int c) { return KV8 ? c / KT : c % KCH; };
  auto ld = [](const __amdgpu_buffer_rsrc_t& r, uint32_t off, uint32_t ch) -> u32x4 {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off == OOB ? OOB : off + ch * 16, 0, 0));
  };
  auto stage_load = [&](auto& kreg, auto& vreg, float& scl, int s0) {
    // per-tile source: compressed keys only, window keys only, or both (the
    // one tile that straddles the boundary); each branch issues its loads back
    // to back
    auto load_all = [&](auto&& fetch) {
#pragma unroll
      for (int i = 0; i < KLD; ++i) {
        const int c = tid + i * NT;
        kreg[i] = fetch(true, c < KT * KCH ? s0 + krow(c) : INT_MAX / 2, kch(c));
      }
#pragma unroll
      for (int i = 0; i < VTK; ++i) {
        const int c = tid + i * NT;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          vreg[i][u] = fetch(false, c < VTOT ? s0 + (c / KCH) * 4 + u : INT_MAX / 2, c % KCH);
      }
    };
    if constexpr (KV8) {
      // FP8 rows: a K chunk below DN dims is 8 codes, above it 8 bf16 RoPE
      // values (the chunk kind is uniform over a wave); a V chunk is 8 codes.
      // Window rows are bf16.  (Values shared with keys: the value row is the
      // key row.)  Threads 0..KT-1 load the key row scale of slot s0 + tid,
      // threads KT..2KT-1 the value row scale (absent rows read 0).
      if (tid < 2 * KT) {
        const int e = ent(s0 + tid % KT);
        const bool vs = tid >= KT && !vshared;
        scl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vs ? rvs : rks, e >= 0 ? (uint32_t)e * 4 : OOB, 0, 0));
      }
      auto comp8 = [&](bool k, int s, int ch) -> u32x4 {
        const int e = ent(s);
        if ((k || vshared) && ch >= DN / VEC) return ld(rkr, e >= 0 ? (uint32_t)e * (D - DN) * 2 : OOB, ch - DN / VEC);
        if (k || vshared) return ld8(rk8, e, (uint32_t)e * DN + ch * 8);
        return ld8(rv8, e, (uint32_t)e * D + ch * 8);
      };
      if (s0 + KT <= ncomp || nwin == 0)
        load_all(comp8);
      else if (s0 >= ncomp)
        load_all([&](bool k, int s, int ch) { return ld(k ? rkw : rvw, win_off(s), ch); });
      else
        load_all([&](bool k, int s, int ch) { return comp8(k, s, ch) | ld(k ? rkw : rvw, win_off(s), ch); });
    } else if (s0 + KT <= ncomp && s0 + KT <= kend) {
      // every slot of the tile holds a compressed entry of this split: row
      // offsets straight from the entry (sparse: from the index list, an
      // invalid entry giving an out-of-range offset, read as zeros and masked
      // in the softmax), without the per-slot range checks
      auto eoff = [&](int e) -> uint32_t { return (e >= 0 && e < a.Nc_cap) ? (uint32_t)e * ROWB : OOB; };
#pragma unroll
      for (int i = 0; i < KLD; ++i) {
        const int c = tid + i * NT;
        const int s = s0 + krow(c);
        int e = s;
        if constexpr (SPARSE) e = c < KT * KCH ? sel[s - sel_base] : -1;
        kreg[i] = ld(rkc, c < KT * KCH ? eoff(e) : OOB, kch(c));
      }
#pragma unroll
      for (int i = 0; i < VTK; ++i) {
        const int c = tid + i * NT;
        const int s = s0 + (c / KCH) * 4;                    // four consecutive slots
        int e4[4] = {s, s + 1, s + 2, s + 3};
        if constexpr (SPARSE) {
          if (c < VTOT) {
            const int4 v = *reinterpret_cast<const int4*>(sel + (s - sel_base));
            e4[0] = v.x; e4[1] = v.y; e4[2] = v.z; e4[3] = v.w;
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) vreg[i][u] = ld(rvc, c < VTOT ? eoff(e4[u]) : OOB, c % KCH);
      }
    } else if (s0 + KT <= ncomp || nwin == 0) {
      load_all([&](bool k, int s, int ch) { return ld(k ? rkc : rvc, comp_off(s), ch); });
    } else if (s0 >= ncomp) {
      load_all([&](bool k, int s, int ch) { return ld(k ? rkw : rvw, win_off(s), ch); });
    } else {
      load_all([&](bool k, int s, int ch) {
        return ld(k ? rkc : rvc, comp_off(s), ch) | ld(k ? rkw : rvw, win_off(s), ch);
      });
    }
  };
  auto stage_store = [&](const auto& kreg, const auto& vreg, float scl, int s0) {
    if constexpr (KV8) {
      // row scales of the tile's keys; 1 for window rows (bf16, unscaled)
      if (tid < 2 * KT) (tid < KT ? kscl : vscl)[tid % KT] = ent(s0 + tid % KT) >= 0 ? scl : 1.f;
    }
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int c = tid + i * NT;
      if (c >= KT * KCH) continue;
      u32x4 r = kreg[i];
      if constexpr (KV8)
        if (kch(c) < DN / VEC && ent(s0 + krow(c)) >= 0) r = widen8(r);
      *reinterpret_cast<u32x4*>(Ks + krow(c) * KS + kch(c) * VEC) = r;
    }
#pragma unroll
    for (int i = 0; i < VTK; ++i) {
      const int c = tid + i * NT;
      if (c >= VTOT) continue;
      const int kg = c / KCH, ch = c % KCH;
      u32x4 vr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        vr[u] = vreg[i][u];
        if constexpr (KV8)
          if ((!vshared || ch < DN / VEC) && ent(s0 + kg * 4 + u) >= 0) vr[u] = widen8(vr[u]);
      }
      if constexpr (sizeof(T) == 2) {
        // dim ch*8+e of the four keys: 16-bit half e&1 of word e>>1 of each
        // row, paired by byte permutes; the 8 dims share one swizzled block
        // (vt_block depends on the dim's 8-group only), 8 rows apart
        T* dst = Vt + ch * VEC * VS + vt_block(ch * VEC, kg) * 4;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t w01 = __builtin_amdgcn_perm(vr[1][e >> 1], vr[0][e >> 1], sel);
          const uint32_t w23 = __builtin_amdgcn_perm(vr[3][e >> 1], vr[2][e >> 1], sel);
          *reinterpret_cast<uint2*>(dst + e * VS) = uint2{w01, w23};
        }
      } else {
        const T* rows = reinterpret_cast<const T*>(vr);         // [4][VEC]
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          T four[4] = {rows[e], rows[VEC + e], rows[2 * VEC + e], rows[3 * VEC + e]};
          T* dst = Vt + (ch * VEC + e) * VS + vt_block(ch * VEC + e, kg) * 4;
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<u32x4*>(four);
        }
      }
    }
  };

  if (kbeg < kend) stage_load(kregA, vregA, sclA, kbeg);
  if constexpr (PF == 2) {
    if (kbeg + KT < kend) stage_load(kregB, vregB, sclB, kbeg + KT);
  }
  // One tile ahead: the first staging store needs the first tile, so waiting
  // here for every load (the query fragments included) costs nothing, and it
  // tells the compiler's wait insertion that the query registers are ready,
  // so the loop does not wait on the vector-memory counter at the query's
  // uses (which, in steady state, would hold the MFMAs until the next tile's
  // prefetch had landed).
  if constexpr (PF == 1) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  // the row scales of a lane's 16 keys in sub-tile `sub` (S^T rows
  // 8 (r >> 2) + 4 half + (r & 3)), from the staged scale array
  auto lane_scales = [&](const float* scl_arr, int sub, float (&out)[16]) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(scl_arr + sub * 32 + 8 * g4 + 4 * half);
#pragma unroll
      for (int u = 0; u < 4; ++u) out[4 * g4 + u] = v[u];
    }
  };

  auto tile = [&](int s0) {
    // ---- S^T = K Q^T for this wave's 32-key sub-tiles ----
    // (FP8 caches: the dims below DN hold unscaled codes; their partial dot
    // products are accumulated first and multiplied by the key row scale in
    // fp32 before the RoPE dims are added)
    f32x16 st[NSUB];
#pragma unroll
    for (int si = 0; si < NSUB; ++si)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[si][r] = 0.f;
#pragma unroll
    for (int s = 0; s < DSTEP; ++s) {
      if constexpr (KV8) {
        if (16 * s == DN) {
#pragma unroll
          for (int si = 0; si < NSUB; ++si) {
            float ks[16];
            lane_scales(kscl, KG == 2 ? kg : si, ks);
#pragma unroll
            for (int r = 0; r < 16; ++r) st[si][r] *= ks[r];
          }
        }
      }
#pragma unroll
      for (int si = 0; si < NSUB; ++si) {
        const int sub = KG == 2 ? kg : si;
        Frag<T> kf;
        frag_load(kf, Ks + (sub * 32 + col) * KS + 16 * s + 8 * half);
        mma32(st[si], kf, qfr[s]);
      }
    }
    // ---- mask (only tiles that reach a boundary), online softmax ----
    const int t_end = s0 + KT;
    bool comp_ok = true;                       // every compressed slot of the tile holds an entry
    if constexpr (SPARSE) {
      if (sel_base > 0 || gm.nsplit > 1) {
        const int sl = s0 + lane;
        const int e = sl < min(t_end, ncomp) ? sel[sl - sel_base] : 0;
        comp_ok = __all(e >= 0 && e < a.Nc_cap);
      }
    }
    const bool full = t_end <= kend &&
                      (SPARSE ? comp_ok && (t_end <= ncomp || win_ok) : (t_end <= ncomp && t_end <= wave_min_ne));
    float mt = -INFINITY;
#pragma unroll
    for (int si = 0; si < NSUB; ++si) {
      const int sub = KG == 2 ? kg : si;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = st[si][r];                   // raw q.k; the scale is applied in the exponent
        if (!full) {
          const int s = s0 + sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          bool ok = qvalid && s < kend;
          if (ok && s >= ncomp) {
            const int p = wlo + (s - ncomp);
            ok = (p - rp0 >= 0) && (p - rp0 < a.R) && (kwb != nullptr);   // row present
            if (!SPARSE) ok = ok && p >= q_wlo && p <= qpos;
          } else if (ok) {
            if constexpr (SPARSE) {
              const int e = sel[s - sel_base];
              ok = e >= 0 && e < a.Nc_cap;
            } else {
              ok = s < q_ne;
            }
          }
          x = ok ? x : -INFINITY;
        }
        st[si][r] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * gm.scale_log2;   // scale > 0 keeps the order
    // The reference max only moves when a lane's tile max exceeds it by more
    // than 8 (log2 units): P stays <= 2^8 and most tiles skip the O rescale.
    if (__any(mt > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == -INFINITY) ? 1.f : fexp2<T>(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DVT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
    // P for the value dims; FP8 caches: P times the value row scale for the
    // code dims (pf), and, when values are the key rows, plain P for their
    // bf16 RoPE dims (pr).  A lane's 16 values of a 32-key sub-tile are keys
    // 8 (r >> 2) + 4 half + (r & 3); fragment g of the sub-tile takes the
    // 4-key runs r = 4g..4g+3 and 8+4g..8+4g+3 (keys 4 half + 8g and
    // 16 + 4 half + 8g), which are the two V blocks one paired LDS read brings.
    // For odd dv tiles the swizzle puts the ks = 1 block of a pair below the
    // ks = 0 block, so those tiles take the pair in address order and the
    // fragments in the matching order (pfs; plain caches only).
    constexpr bool SWAPF = !KV8;
    Frag<T> pf[NSUB][2], pr[VSH ? NSUB : 1][2], pfs[SWAPF ? NSUB : 1][2];
    auto split_frags = [](Frag<T> (&f)[2], const float* x, bool swap) {
      float a[8], c[8];
      const int lo = swap ? 8 : 0, hi = swap ? 0 : 8;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = x[lo + u];
        a[4 + u] = x[hi + u];
        c[u] = x[lo + 4 + u];
        c[4 + u] = x[hi + 4 + u];
      }
      frag_from_f32(f[0], a);
      frag_from_f32(f[1], c);
    };
#pragma unroll
    for (int si = 0; si < NSUB; ++si) {
      float pv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = fexp2<T>(fmaf(st[si][r], gm.scale_log2, -m_use));
        psum += pv[r];
      }
      if constexpr (KV8) {
        float vs[16], pw[16];
        lane_scales(VSH ? kscl : vscl, KG == 2 ? kg : si, vs);
#pragma unroll
        for (int r = 0; r < 16; ++r) pw[r] = pv[r] * vs[r];
        split_frags(pf[si], pw, false);
        if constexpr (VSH) split_frags(pr[si], pv, false);
      } else {
        split_frags(pf[si], pv, false);
        split_frags(pfs[si], pv, true);
      }
    }
    l_run += psum;

    // ---- O^T += V^T P^T ----
    // Lane (col, half) reads dim row 32i + col, 4-key blocks kb/4 and kb/4 + 2
    // with kb/4 = 8 sub + 4 ks + half.  The row's swizzle term (row >> 3) is
    // 4i + (col >> 3), so the block position splits into a per-lane part
    // (bits 0-1: (2 hi + half) ^ (col >> 3)) and a part fixed by (i, sub, ks)
    // (bits 2-3: (2 sub + ks) ^ i): two base addresses per lane and
    // immediate offsets address every read.  Fragment g pairs the blocks of
    // ks = 0 and 1 read from base g, so each read pair fills its operand.
    const int c3 = col >> 3;
    const T* vb[2] = {Vt + col * VS + 4 * ((half) ^ c3), Vt + col * VS + 4 * ((2 + half) ^ c3)};
#pragma unroll
    for (int i = 0; i < DVT; ++i) {
#pragma unroll
      for (int si = 0; si < NSUB; ++si) {
        const int sub = KG == 2 ? kg : si;
        const int off0 = 32 * i * VS + 16 * ((2 * sub) ^ i);
        const int off1 = 32 * i * VS + 16 * ((2 * sub + 1) ^ i);
        const bool sw = SWAPF && (i & 1);                  // compile-time after unrolling
        const int oa = sw ? off1 : off0, oc = sw ? off0 : off1;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          Frag<T> vf;
          if constexpr (sizeof(T) == 2) {
            const uint2 a = *reinterpret_cast<const uint2*>(vb[g] + oa);
            const uint2 c = *reinterpret_cast<const uint2*>(vb[g] + oc);
            vf.v = u32x4{a.x, a.y, c.x, c.y};
          } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(vb[g] + oa);
            const f32x4 c = *reinterpret_cast<const f32x4*>(vb[g] + oc);
            float* fv = reinterpret_cast<float*>(&vf);
            fv[0] = a[0]; fv[1] = a[1]; fv[2] = a[2]; fv[3] = a[3];
            fv[4] = c[0]; fv[5] = c[1]; fv[6] = c[2]; fv[7] = c[3];
          }
          if constexpr (VSH) mma32(o[i], vf, 32 * i >= DN ? pr[si][g] : pf[si][g]);
          else if constexpr (SWAPF) mma32(o[i], vf, sw ? pfs[si][g] : pf[si][g]);
          else mma32(o[i], vf, pf[si][g]);
        }
      }
    }
  };
  if constexpr (PF == 2) {
    for (int s0 = kbeg; s0 < kend; s0 += 2 * KT) {
      stage_store(kregA, vregA, sclA, s0);
      __syncthreads();
      if (s0 + 2 * KT < kend) stage_load(kregA, vregA, sclA, s0 + 2 * KT);
      tile(s0);
      __syncthreads();
      if (s0 + KT >= kend) break;
      stage_store(kregB, vregB, sclB, s0 + KT);
      __syncthreads();
      if (s0 + 3 * KT < kend) stage_load(kregB, vregB, sclB, s0 + 3 * KT);
      tile(s0 + KT);
      __syncthreads();
    }
  } else if constexpr (DB) {
    // Two key-tile buffers: tile j is computed from buffer j & 1 while tile
    // j + 1 is staged into the other, so one barrier per tile suffices (it
    // publishes tile j + 1 and frees buffer j & 1 for tile j + 2).  The
    // second half of the waves stages the next tile before computing, the
    // first half after: each SIMD holds one wave of each half, so one wave's
    // staging work runs beside the other's MFMAs.
    T* const k0 = Ks;
    T* const v0 = Vt;
    const bool early = wave >= NW / 2;
    if (kbeg < kend) {
      stage_store(kregA, vregA, sclA, kbeg);
      if (kbeg + KT < kend) stage_load(kregA, vregA, sclA, kbeg + KT);
    }
    __syncthreads();
    // the loop is unrolled over the two buffers so that each half addresses
    // its buffer with compile-time offsets
    auto step = [&](int s0, auto buf) {
      constexpr int cur = decltype(buf)::value;
      auto stage_next = [&]() {
        if (s0 + KT < kend) {
          Ks = k0 + (cur ^ 1) * DBUF;
          Vt = v0 + (cur ^ 1) * DBUF;
          stage_store(kregA, vregA, sclA, s0 + KT);
          if (s0 + 2 * KT < kend) stage_load(kregA, vregA, sclA, s0 + 2 * KT);
        }
      };
      if (early) stage_next();
      Ks = k0 + cur * DBUF;
      Vt = v0 + cur * DBUF;
      tile(s0);
      if (!early) stage_next();
      __syncthreads();
    };
    for (int s0 = kbeg; s0 < kend; s0 += 2 * KT) {
      step(s0, std::integral_constant<int, 0>{});
      if (s0 + KT >= kend) break;
      step(s0 + KT, std::integral_constant<int, 1>{});
    }
  } else {
    for (int s0 = kbeg; s0 < kend; s0 += KT) {
      stage_store(kregA, vregA, sclA, s0);
      __syncthreads();
      if (s0 + KT < kend) stage_load(kregA, vregA, sclA, s0 + KT);
      tile(s0);
      __syncthreads();
    }
  }

  // ---- merge the two key groups (their staging area is free now) ----
  if constexpr (KG == 2) {
    float* mb = reinterpret_cast<float*>(smem_raw) + (size_t)(rw * 64 + lane) * (DVT * 16 + 2);
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < DVT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) mb[i * 16 + r] = o[i][r];
      mb[DVT * 16] = m_run;
      mb[DVT * 16 + 1] = l_run;
    }
    __syncthreads();
    if (kg == 1) return;
    const float m1 = mb[DVT * 16], l1 = mb[DVT * 16 + 1];
    const float M = fmaxf(m_run, m1);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    const float c0 = fexp2<T>(m_run - Mu), c1 = fexp2<T>(m1 - Mu);
#pragma unroll
    for (int i = 0; i < DVT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] = o[i][r] * c0 + mb[i * 16 + r] * c1;
    l_run = l_run * c0 + l1 * c1;
    m_run = M;
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  const size_t grow = ((size_t)b * a.Tq + tq) * a.H + hq;
  if (gm.nsplit > 1) {
    // split partial: o (unnormalised, in the element type: bf16 problems keep
    // bf16 partials, which halves the partials' HBM round trip), max, sum
    const size_t rows_total = (size_t)a.B * a.Tq * a.H;
    T* po = reinterpret_cast<T*>(a.ws) + ((size_t)split * rows_total + grow) * D;
    float* pm = reinterpret_cast<float*>(a.ws) + (size_t)gm.nsplit * rows_total * D;
    float* pl = pm + (size_t)gm.nsplit * rows_total;
#pragma unroll
    for (int i = 0; i < DVT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T* dst = po + i * 32 + 8 * g + 4 * half;
        if constexpr ((COH & COH_PART) != 0) {
          if constexpr (sizeof(T) == 2) {
            const uint64_t v = (uint64_t)pack_bf16x2(o[i][4 * g], o[i][4 * g + 1]) |
                               ((uint64_t)pack_bf16x2(o[i][4 * g + 2], o[i][4 * g + 3]) << 32);
            __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              __hip_atomic_store(reinterpret_cast<uint32_t*>(dst) + u, __float_as_uint(o[i][4 * g + u]),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        } else if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(dst) =
              uint2{pack_bf16x2(o[i][4 * g], o[i][4 * g + 1]), pack_bf16x2(o[i][4 * g + 2], o[i][4 * g + 3])};
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{o[i][4 * g], o[i][4 * g + 1], o[i][4 * g + 2], o[i][4 * g + 3]};
        }
      }
    if (half == 0) {
      if constexpr ((COH & COH_PART) != 0) {
        __hip_atomic_store(reinterpret_cast<uint32_t*>(pm) + (size_t)split * rows_total + grow,
                           __float_as_uint(m_run), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(reinterpret_cast<uint32_t*>(pl) + (size_t)split * rows_total + grow,
                           __float_as_uint(l_tot), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        pm[(size_t)split * rows_total + grow] = m_run;
        pl[(size_t)split * rows_total + grow] = l_tot;
      }
    }
    return;
  }
  const float s2 = a.sink ? a.sink[hq] * LOG2E : -INFINITY;
  const float M = fmaxf(m_run, s2);
  float fac = 0.f, lse = -INFINITY;
  if (M != -INFINITY) {
    const float cm = fexp2<T>(m_run - M);             // m_run = -inf -> 0
    const float Z = l_tot * cm + fexp2<T>(s2 - M);
    fac = cm / Z;
    lse = (M + __log2f(Z)) * LN2;
  }
  T* orow = reinterpret_cast<T*>(a.out) + grow * D;
#pragma unroll
  for (int i = 0; i < DVT; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      T v4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v4[u] = from_f32<T>(o[i][4 * g + u] * fac);
      T* dst = orow + i * 32 + 8 * g + 4 * half;
      if constexpr (sizeof(T) == 2) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<uint2*>(v4);
      else *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<u32x4*>(v4);
    }
  if (a.lse && half == 0) a.lse[grow] = lse;
}

template <typename T, int D, int RW, int KG, bool SPARSE, int PF, bool KV8, bool VSH>
__global__ __launch_bounds__(RW * KG * 64) __attribute__((amdgpu_waves_per_eu(KV8 && !(RW == 2 && KG == 2) ? 1 : 2))) void attend_kernel(AttendArgs a, AttnGeom gm) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int gx = (a.Tq + gm.TT - 1) / gm.TT;
  const RowJ rj = xcd_rows(blockIdx.x, a.B, gx * gm.nsplit);
  attend_body<T, D, RW, KG, SPARSE, PF, KV8, VSH>(a, gm, rj.j % gx, rj.j / gx, rj.row, smem_raw);
}

// The HCA and CSA attention of one layer pair in a single split-decode launch:
// a 1-D grid whose first nb0 workgroups run the HCA problem a0 and the rest the
// CSA problem a1 (each decomposed as its own (tile, split, sequence) grid, the
// same as in its own launch).  Two workgroups fit a compute unit, so the two
// grids of a decode batch run side by side instead of one after the other.
template <typename T, int D, int RW, int KG>
__global__ __launch_bounds__(RW * KG * 64) __attribute__((amdgpu_waves_per_eu(2))) void attend_pair_kernel(
    AttendArgs a0, AttnGeom g0, AttendArgs a1, AttnGeom g1, int nb0) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  int bid = blockIdx.x;
  if (bid < nb0) {
    const int gx = (a0.Tq + g0.TT - 1) / g0.TT;
    const RowJ rj = xcd_rows(bid, a0.B, gx * g0.nsplit);
    attend_body<T, D, RW, KG, false, 2>(a0, g0, rj.j % gx, rj.j / gx, rj.row, smem_raw);
  } else {
    bid -= nb0;
    const int gx = (a1.Tq + g1.TT - 1) / g1.TT;
    const RowJ rj = xcd_rows(bid, a1.B, gx * g1.nsplit);
    attend_body<T, D, RW, KG, true, 2>(a1, g1, rj.j % gx, rj.j / gx, rj.row, smem_raw);
  }
}

// Merge split partials in fixed split order (one wave per query row).  The
// partials of CB splits are requested together; a running maximum rescales
// the sums between batches, so the result depends only on the split list.
// COH: the partials are read with device-scope (sc1) loads (written in the
// same launch, possibly through another XCD's L2).
template <typename T, int D, bool COH = false>
__device__ __forceinline__ void combine_row(const AttendArgs& a, int nsplit, size_t row) {
  static_assert(!COH || (D / 64) * sizeof(T) == 4 || (D / 64) * sizeof(T) == 8,
                "device-scope partial loads take 4 or 8 bytes per lane");
  constexpr int PER = D / 64;
  constexpr int CB = 32;
  const int lane = threadIdx.x & 63;
  const size_t rows_total = (size_t)a.B * a.Tq * a.H;
  if (row >= rows_total) return;
  const T* po = reinterpret_cast<const T*>(a.ws);               // partials in the element type
  const float* pm = reinterpret_cast<const float*>(a.ws) + (size_t)nsplit * rows_total * D;
  const float* pl = pm + (size_t)nsplit * rows_total;
  const int h = (int)(row % a.H);
  const float s2 = a.sink ? a.sink[h] * LOG2E : -INFINITY;
  float M = s2, Z = 0.f;
  float acc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) acc[u] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += CB) {
    // every load is unconditional (split indices past the end repeat the last
    // split, whose weight is then zero), so all of them are in flight together
    float v[CB][PER];
    const int sl = min(s0 + (lane & (CB - 1)), nsplit - 1);
    const bool lv_ok = lane < CB && s0 + lane < nsplit;
    float mraw, lraw;
    if constexpr (COH) {
      mraw = __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(pm) + (size_t)sl * rows_total + row,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      lraw = __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(pl) + (size_t)sl * rows_total + row,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    } else {
      mraw = pm[(size_t)sl * rows_total + row];
      lraw = pl[(size_t)sl * rows_total + row];
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const T* src = po + ((size_t)min(s0 + j, nsplit - 1) * rows_total + row) * D + lane * PER;
      if constexpr (COH) {
        T t[PER];
        if constexpr (PER * sizeof(T) == 4) {
          const uint32_t w = __hip_atomic_load(reinterpret_cast<const uint32_t*>(src), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          __builtin_memcpy(t, &w, 4);
        } else {
          const uint64_t w = __hip_atomic_load(reinterpret_cast<const uint64_t*>(src), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
          __builtin_memcpy(t, &w, 8);
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) v[j][u] = to_f32(t[u]);
      } else {
#pragma unroll
        for (int u = 0; u < PER; ++u) v[j][u] = to_f32(src[u]);
      }
    }
    const float mv = lv_ok ? mraw : -INFINITY;
    const float lv = lv_ok ? lraw : 0.f;
    const float M_new = fmaxf(M, wave_max(mv));
    if (M_new == -INFINITY) continue;
    const float r = __builtin_amdgcn_exp2f(M - M_new);      // M = -inf -> 0
    Z *= r;
#pragma unroll
    for (int u = 0; u < PER; ++u) acc[u] *= r;
    const float cl = __builtin_amdgcn_exp2f(mv - M_new);     // this lane's split weight
    Z += wave_sum(lv * cl);
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const float c = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(cl), j));
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] = fmaf(v[j][u], c, acc[u]);
    }
    M = M_new;
  }
  float lse = -INFINITY, inv = 0.f;
  if (M != -INFINITY) {
    Z += __builtin_amdgcn_exp2f(s2 - M);
    lse = (M + __log2f(Z)) * LN2;
    inv = 1.f / Z;
  }
  T* orow = reinterpret_cast<T*>(a.out) + row * D;
#pragma unroll
  for (int u = 0; u < PER; ++u) orow[lane * PER + u] = from_f32<T>(acc[u] * inv);
  if (a.lse && lane == 0) a.lse[row] = lse;
}

// The query row merged by wave `wave` of merge workgroup `bid` (4 rows per
// workgroup): the rows of one sequence on that sequence's XCD (xcd_rows),
// where its split workgroups wrote their partials.
__device__ __forceinline__ size_t combine_row_of(const AttendArgs& a, int bid, int wave) {
  const int per = a.Tq * a.H;
  if ((per & 3) == 0) {
    const RowJ rj = xcd_rows(bid, a.B, per >> 2);
    return (size_t)rj.row * per + (size_t)rj.j * 4 + wave;
  }
  return (size_t)bid * 4 + wave;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(AttendArgs a, int nsplit) {
  combine_row<T, D>(a, nsplit, combine_row_of(a, blockIdx.x, threadIdx.x >> 6));
}

// Both problems of a pair launch: workgroups below nb0 merge a0's rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_pair_kernel(AttendArgs a0, int ns0, AttendArgs a1, int ns1,
                                                           int nb0) {
  if ((int)blockIdx.x < nb0) combine_row<T, D>(a0, ns0, combine_row_of(a0, blockIdx.x, threadIdx.x >> 6));
  else combine_row<T, D>(a1, ns1, combine_row_of(a1, blockIdx.x - nb0, threadIdx.x >> 6));
}

// ------------------------- host launch templates ---------------------------
// Instantiated per (element type, head dim, cache format) in the attend_v_*.hip
// translation units; attend.hip dispatches to them.
// Keys per split of a one-token (decode) problem, from the key count only (so
// results never depend on the batch): dense 256; sparse 192 for lists of up
// to 1536 keys (a top-1024 list + window in 6 splits: fewer workgroups and
// partials), 128 beyond (a top-2048 list + window in 17 two-tile splits,
// which stay shorter than the dense problem's in a layer pair's launch).
static inline int keys_per_split(bool sparse, int Tq, long nk) {
  if (Tq != 1) return INT_MAX / 2;
  if (!sparse) return 256;
  return nk <= 1536 ? 192 : 128;
}

// Dense (HCA) prefill tiles of bf16 problems hold up to 256 (token, head)
// rows, so that eight row-waves share every staged key tile (half the
// staging work and LDS writes per MFMA of a 128-row tile); other tiles hold
// up to 128 rows.
static inline int tokens_per_tile(bool sparse, int H, int Tq, bool wide) {
  if (sparse) return 1;
  return std::max(1, std::min((wide ? 256 : 128) / H, Tq));
}

static inline int nkeys_upper(bool sparse, int topk, int window, int Nc_cap, int m_prime, int max_pos) {
  const int w = window > 0 ? std::min(window, max_pos + 1) : 0;
  if (sparse) return topk + w;
  return hca_ne(max_pos, m_prime, Nc_cap) + w;
}

static inline AttnGeom make_geom(const AttendArgs& a) {
  AttnGeom gm;
  gm.TT = tokens_per_tile(a.sparse, a.H, a.Tq, !a.f32 && !a.kv8 && a.Tq > 1);
  const long nk = nkeys_upper(a.sparse, a.topk, a.window, a.Nc_cap, a.m_prime, a.max_pos);
  const int kps = keys_per_split(a.sparse, a.Tq, nk);
  gm.nsplit = (int)std::max(1L, (nk + kps - 1) / kps);
  gm.kps = gm.nsplit > 1 ? kps : INT_MAX / 2;
  gm.scale_log2 = a.scale * LOG2E;
  return gm;
}

// Row-waves cover the tile's (token, head) rows; tiles of at most 64 rows get
// a second key group so that four waves share every staged tile; 256-row
// tiles (dense bf16 prefill) take eight row-waves.
static inline void wave_shape(int rows, int* RW, int* KG) {
  if (rows <= 32) { *RW = 1; *KG = 2; }
  else if (rows <= 64) { *RW = 2; *KG = 2; }
  else if (rows <= 96) { *RW = 3; *KG = 1; }
  else if (rows <= 128) { *RW = 4; *KG = 1; }
  else { *RW = 8; *KG = 1; }
}

static inline size_t partial_rows(const AttendArgs& a) { return (size_t)a.B * a.Tq * a.H; }

// How a split attention is launched: with or without its split merge.
struct AttendLaunch {
  bool combine = true;
};

template <typename T, int D, bool SPARSE>
static size_t attend_lds(const AttendArgs& a, int RW, int KG) {
  constexpr int KS = D + 16 / sizeof(T);
  constexpr int VS = KT + 4;
  // 256-row dense tiles are only formed for prefill (one split, one tile ahead)
  const size_t bufs = attend_double_buffered(SPARSE, a.kv8, RW, 1) ? 2 : 1;
  size_t lds = bufs * (KT * KS + D * VS) * sizeof(T) + (SPARSE ? (size_t)a.topk * 4 : 0) +
               (a.kv8 ? 2 * KT * sizeof(float) : 0);
  if (KG == 2) lds = std::max(lds, (size_t)RW * 64 * ((D / 32) * 16 + 2) * sizeof(float));
  return lds;
}

template <typename K>
static hipError_t set_lds(K kfn, size_t lds) {
  return ensure_lds_limit((const void*)kfn, lds);
}

template <typename T, int D, int RW, int KG, bool SPARSE, int PF, bool KV8, bool VSH>
static hipError_t launch5(const AttendArgs& a, const AttnGeom& gm, const AttendLaunch& how, hipStream_t st) {
  const size_t lds = attend_lds<T, D, SPARSE>(a, RW, KG);
  auto kfn = attend_kernel<T, D, RW, KG, SPARSE, PF, KV8, VSH>;
  hipError_t e = set_lds(kfn, lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((a.Tq + gm.TT - 1) / gm.TT * gm.nsplit * a.B));
  {
    ProfScope ps(SPARSE ? "attend_csa" : "attend_hca", st);
    hipLaunchKernelGGL(kfn, grid, dim3(RW * KG * 64), lds, st, a, gm);
  }
  e = hipGetLastError();
  if (e != hipSuccess || gm.nsplit <= 1 || !how.combine) return e;
  ProfScope ps("attend_combine", st);
  hipLaunchKernelGGL((combine_kernel<T, D>), dim3((unsigned)((partial_rows(a) + 3) / 4)), dim3(256), 0, st,
                     a, gm.nsplit);
  return hipGetLastError();
}

template <typename T, int D, int RW, int KG, bool SPARSE, bool KV8>
static hipError_t launch4(const AttendArgs& a, const AttnGeom& gm, const AttendLaunch& how, hipStream_t st) {
  if constexpr (KV8) {
    // FP8 caches keep one tile in flight ahead also in split decode: with two
    // the staging registers pushed the kernel past 256 registers, and its
    // spill reloads waited for every load in flight
    if (a.v8 == nullptr)                     // values are the key rows
      return launch5<T, D, RW, KG, SPARSE, 1, true, true>(a, gm, how, st);
    return launch5<T, D, RW, KG, SPARSE, 1, true, false>(a, gm, how, st);
  }
  return gm.nsplit > 1 ? launch5<T, D, RW, KG, SPARSE, 2, KV8, false>(a, gm, how, st)
                       : launch5<T, D, RW, KG, SPARSE, 1, KV8, false>(a, gm, how, st);
}

template <typename T, int D, bool SPARSE, bool KV8>
static hipError_t launch3(const AttendArgs& a, const AttnGeom& gm, const AttendLaunch& how, hipStream_t st) {
  int RW, KG;
  wave_shape(gm.TT * a.H, &RW, &KG);
  if (RW == 1) return launch4<T, D, 1, 2, SPARSE, KV8>(a, gm, how, st);
  if (RW == 2) return launch4<T, D, 2, 2, SPARSE, KV8>(a, gm, how, st);
  if (RW == 3) return launch4<T, D, 3, 1, SPARSE, KV8>(a, gm, how, st);
  if (RW == 4) return launch4<T, D, 4, 1, SPARSE, KV8>(a, gm, how, st);
  // 256-row tiles are formed only for dense bf16 prefill problems
  if constexpr (!SPARSE && !KV8 && sizeof(T) == 2) return launch4<T, D, 8, 1, SPARSE, KV8>(a, gm, how, st);
  return hipErrorInvalidValue;
}

// One attention problem (its kernel, and its split merge if asked).
template <typename T, int D, bool KV8>
hipError_t attend_variant(const AttendArgs& a, const AttnGeom& gm, const AttendLaunch& how, hipStream_t st) {
  return a.sparse ? launch3<T, D, true, KV8>(a, gm, how, st) : launch3<T, D, false, KV8>(a, gm, how, st);
}

// The split partials of a CSA problem c and an HCA problem h merged in one launch.
template <typename T, int D>
hipError_t combine_pair_variant(const AttendArgs& h, const AttnGeom& gh, const AttendArgs& c,
                                const AttnGeom& gc, hipStream_t st) {
  const long cbh = (long)((partial_rows(h) + 3) / 4), cbc = (long)((partial_rows(c) + 3) / 4);
  ProfScope ps("attend_combine", st);
  hipLaunchKernelGGL((combine_pair_kernel<T, D>), dim3((unsigned)(cbh + cbc)), dim3(256), 0, st,
                     h, gh.nsplit, c, gc.nsplit, (int)cbh);
  return hipGetLastError();
}

template <typename T, int D, int RW, int KG>
static hipError_t launch_pair4(const AttendArgs& h, const AttnGeom& gh, const AttendArgs& c,
                               const AttnGeom& gc, hipStream_t st) {
  const size_t lds = std::max(attend_lds<T, D, false>(h, RW, KG), attend_lds<T, D, true>(c, RW, KG));
  auto kfn = attend_pair_kernel<T, D, RW, KG>;
  hipError_t e = set_lds(kfn, lds);
  if (e != hipSuccess) return e;
  const long nbh = (long)((h.Tq + gh.TT - 1) / gh.TT) * gh.nsplit * h.B;
  const long nbc = (long)((c.Tq + gc.TT - 1) / gc.TT) * gc.nsplit * c.B;
  {
    ProfScope ps("attend_pair", st);
    hipLaunchKernelGGL(kfn, dim3((unsigned)(nbh + nbc)), dim3(RW * KG * 64), lds, st, h, gh, c, gc, (int)nbh);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return combine_pair_variant<T, D>(h, gh, c, gc, st);
}

// Both problems of a layer pair in one kernel (shapes checked by the caller).
template <typename T, int D>
hipError_t pair_variant(const AttendArgs& h, const AttnGeom& gh, const AttendArgs& c,
                        const AttnGeom& gc, int RW, hipStream_t st) {
  if (RW == 1) return launch_pair4<T, D, 1, 2>(h, gh, c, gc, st);
  if (RW == 2) return launch_pair4<T, D, 2, 2>(h, gh, c, gc, st);
  if (RW == 3) return launch_pair4<T, D, 3, 1>(h, gh, c, gc, st);
  return launch_pair4<T, D, 4, 1>(h, gh, c, gc, st);
}

}  // namespace csa
