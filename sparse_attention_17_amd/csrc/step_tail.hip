// The tail of one hybrid decode step in a single launch: the top-k pick of
// every CSA query row, the HCA and CSA split attention, and the merges of both
// problems' split partials, with the dependencies between them resolved inside
// the kernel instead of by kernel boundaries.
// Method: DeepSeek-V4 summary (hyper.ai), "Method": CSA keeps the top-k
// compressed entries chosen by the lightning indexer and attends over them
// plus a sliding window; HCA attends densely over its compressed entries.
// research.elamur.ai, "Key points" (infrastructure: batch-invariant,
// deterministic kernels) and the git.lyz.one wiki, "Infrastructure Highlights"
// (fused kernels): every task computes exactly what the separate kernels do,
// in the same order, so the results are bitwise those of the multi-launch step.
//
// Work distribution (MI355X: 8 XCDs, workgroups dealt round-robin):
//   * sequence b belongs to queue b mod 8 when the batch is a multiple of 8
//     (one queue otherwise), and workgroup i serves queue i mod 8, so all of a
//     sequence's tasks run on the XCD whose L2 holds its candidates and
//     partials;
//   * a workgroup takes the next task of its queue from an atomic counter, so
//     a task only ever waits on tasks fetched before it, which are resident or
//     finished: the waits cannot deadlock;
//   * queue order: picks, HCA splits (no dependencies: they run while the
//     picks are in progress), CSA splits (wait for their row's pick), HCA
//     merges (wait for the sequence's HCA splits), CSA merges (wait for its
//     CSA splits);
//   * data passes through global memory with device-scope (sc1) stores and
//     loads, which bypass the per-XCD caches' incoherence, and counters
//     updated after the writer's stores have completed; every wait is bounded
//     in time and, past the bound, sets an abort flag that ends all waits
//     (results are then undefined and the event is counted).
// Control words live at the front of the workspace: zero before the first
// launch, and every launch returns them to zero (each counter is reset by the
// last task that reads it).
#include "attend_impl.hpp"
#include "pick_impl.hpp"
#include "step_tail.hpp"

namespace csa {

namespace {

constexpr int CTL_FETCH = 0;          // queue q's task counter at word 32 q (own cache line)
constexpr int CTL_ABORT = 256;        // set when a wait runs out of time
constexpr int CTL_ROWS = 288;         // five per-sequence arrays follow
// The control block has one fixed size whatever the batch, so that the rest
// of the workspace never overlaps words another call uses as counters.
constexpr int CTL_WORDS = 8192;
constexpr int TAIL_MAX_B = (CTL_WORDS - CTL_ROWS) / 5;
constexpr long long WAIT_TICKS = 50000000;   // 0.5 s of the 100 MHz real-time counter

struct TailArgs {
  IndexerArgs ix;
  AttendArgs h, c;
  AttnGeom gh, gc;
  uint32_t* ctl;
  unsigned long long* counters;
  int nq;       // queues: 8 (batch a multiple of 8) or 1
  int len;      // tasks per queue (the grid holds nq * len workgroups)
  int mt;       // merge tasks per sequence and problem (4 query rows each)
  int picks;    // 1: the row picks are tasks of this launch (else done before it)
};

struct SeqCtl {
  uint32_t *pick, *csplit, *hsplit, *cmerge, *hmerge;
};
__device__ __forceinline__ SeqCtl seq_ctl(uint32_t* ctl, int B, int b) {
  uint32_t* r = ctl + CTL_ROWS;
  return SeqCtl{r + b, r + B + b, r + 2 * B + b, r + 3 * B + b, r + 4 * B + b};
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish this workgroup's results, then add 1 to *p; returns the previous
// value (to every thread).  Everything another workgroup of the launch reads
// (index rows, split partials) was stored with device scope (sc1), so waiting
// for this wave's stores to complete is the whole release: no cache write-back
// is needed (on gfx950 an agent-scope fence writes back the XCD's whole L2).
__device__ __forceinline__ uint32_t signal_add(uint32_t* p, uint32_t* s_word) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) *s_word = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *s_word;
}

// Wait until *p >= target.  One lane polls (device-scope loads); the data the
// waiting task then reads is loaded with device scope too, so no cache
// invalidation is needed.  The wait ends early once the abort flag is set, and
// sets it (counting the event) past WAIT_TICKS.
__device__ __forceinline__ void wait_geq(const TailArgs& t, const uint32_t* p, uint32_t target) {
  if (threadIdx.x == 0) {
    const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
    while (ld_agent(p) < target) {
      if (ld_agent(t.ctl + CTL_ABORT) != 0u) break;
      if ((long long)__builtin_amdgcn_s_memrealtime() - t0 > WAIT_TICKS) {
        st_agent(t.ctl + CTL_ABORT, 1u);
        count_event_at(t.counters, CNT_STEP_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

}  // namespace

template <typename T, int D, int RW, int KG>
__global__ __launch_bounds__(RW * KG * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_tail_kernel(TailArgs t) {
  static_assert(RW * KG * 64 == 256, "the pick runs on 256-thread workgroups");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ uint32_t s_word;
  const int q = t.nq == 8 ? (int)(blockIdx.x & 7u) : 0;
  if (threadIdx.x == 0) {
    uint32_t* fetch = t.ctl + CTL_FETCH + 32 * q;
    const uint32_t v = __hip_atomic_fetch_add(fetch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v == (uint32_t)t.len - 1) st_agent(fetch, 0u);       // the queue's last fetch
    s_word = v;
  }
  __syncthreads();
  if (s_word >= (uint32_t)t.len) {                           // control words not zero at launch
    if (threadIdx.x == 0) count_event_at(t.counters, CNT_STEP_TIMEOUT);
    return;
  }
  int i = (int)s_word;
  const int B = t.c.B, H = t.c.H;
  const int nbq = (B - q + t.nq - 1) / t.nq;                 // sequences q, q + nq, ...
  const int HS = t.gh.nsplit, CS = t.gc.nsplit, MT = t.mt;
  const int wave = threadIdx.x >> 6;
  const int np = t.picks ? nbq : 0;

  if (i < np) {                                              // top-k pick of one row
    const int b = q + t.nq * i;
    pick_row<256>(*reinterpret_cast<PickSmem<256>*>(smem_raw), t.ix, b, t.counters);
    signal_add(seq_ctl(t.ctl, B, b).pick, &s_word);
    return;
  }
  i -= np;
  if (i < nbq * HS) {                                        // HCA split
    const int b = q + t.nq * (i / HS);
    attend_body<T, D, RW, KG, false, 2, false, false, COH_PART>(t.h, t.gh, 0, i % HS, b, smem_raw);
    signal_add(seq_ctl(t.ctl, B, b).hsplit, &s_word);
    return;
  }
  i -= nbq * HS;
  if (i < nbq * CS) {                                        // CSA split, after its row's pick
    const int b = q + t.nq * (i / CS);
    const SeqCtl s = seq_ctl(t.ctl, B, b);
    if (t.picks) {
      wait_geq(t, s.pick, 1u);
      attend_body<T, D, RW, KG, true, 2, false, false, COH_IDX | COH_PART>(t.c, t.gc, 0, i % CS, b, smem_raw);
    } else {
      attend_body<T, D, RW, KG, true, 2, false, false, COH_PART>(t.c, t.gc, 0, i % CS, b, smem_raw);
    }
    signal_add(s.csplit, &s_word);
    return;
  }
  i -= nbq * CS;
  if (i < 2 * nbq * MT) {                                    // merges: HCA, then CSA
    const bool hca = i < nbq * MT;
    if (!hca) i -= nbq * MT;
    const int b = q + t.nq * (i / MT), part = i % MT;
    const SeqCtl s = seq_ctl(t.ctl, B, b);
    const AttendArgs& a = hca ? t.h : t.c;
    wait_geq(t, hca ? s.hsplit : s.csplit, (uint32_t)(hca ? HS : CS));
    const int h = 4 * part + wave;
    if (h < H) combine_row<T, D, true>(a, hca ? HS : CS, (size_t)b * H + h);
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t done = __hip_atomic_fetch_add(hca ? s.hmerge : s.cmerge, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (done == (uint32_t)MT - 1) {                        // the sequence's last merge of this problem
        if (hca) {
          st_agent(s.hsplit, 0u);
          st_agent(s.hmerge, 0u);
        } else {
          st_agent(s.csplit, 0u);
          st_agent(s.cmerge, 0u);
          if (t.picks) st_agent(s.pick, 0u);
        }
      }
    }
  }
}

// ------------------------------- host side --------------------------------
size_t decode_tail_ctl_bytes() { return (size_t)CTL_WORDS * 4; }

bool decode_tail_supported(const AttendArgs& c, const AttendArgs& h) {
  if (c.B <= 0 || c.B > TAIL_MAX_B || c.Tq != 1 || h.Tq != 1 || h.B != c.B || h.H != c.H) return false;
  if (c.f32 || h.f32 || c.kv8 || h.kv8 || c.d != 128 || h.d != 128) return false;
  if (!c.sparse || h.sparse) return false;
  const AttnGeom gc = make_geom(c), gh = make_geom(h);
  if (gc.nsplit <= 1 || gh.nsplit <= 1) return false;
  int rwc, kgc, rwh, kgh;
  wave_shape(gc.TT * c.H, &rwc, &kgc);
  wave_shape(gh.TT * h.H, &rwh, &kgh);
  return rwc == 2 && rwh == 2 && kgc == 2 && kgh == 2;       // 256-thread workgroups

}

static hipError_t launch_tail(TailArgs& t, hipStream_t st) {
  constexpr int RW = 2;
  auto kfn = decode_tail_kernel<bf16, 128, RW, 2>;
  const size_t lds = std::max({sizeof(PickSmem<256>), attend_lds<bf16, 128, false>(t.h, RW, 2),
                               attend_lds<bf16, 128, true>(t.c, RW, 2)});
  hipError_t e = ensure_lds_limit((const void*)kfn, lds);
  if (e != hipSuccess) return e;
  ProfScope ps("decode_tail", st);
  hipLaunchKernelGGL(kfn, dim3((unsigned)(t.nq * t.len)), dim3(RW * 2 * 64), lds, st, t);
  return hipGetLastError();
}

hipError_t launch_decode_tail(const IndexerArgs& ix, const AttendArgs& c, const AttendArgs& h, void* ctl,
                              unsigned long long* counters, bool picks, hipStream_t st) {
  TailArgs t;
  t.ix = ix;
  t.c = c;
  t.h = h;
  t.gc = make_geom(c);
  t.gh = make_geom(h);
  t.ctl = reinterpret_cast<uint32_t*>(ctl);
  t.counters = counters;
  t.nq = (c.B % 8) == 0 ? 8 : 1;
  t.mt = (c.H + 3) / 4;
  t.picks = picks ? 1 : 0;
  const int nbq = (c.B + t.nq - 1) / t.nq;
  t.len = nbq * (t.picks + t.gh.nsplit + t.gc.nsplit + 2 * t.mt);
  return launch_tail(t, st);
}

}  // namespace csa
