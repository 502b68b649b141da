// Grouped output projection after the core attention.
// Method: DeepSeek-V4 summary (hyper.ai), "Method", CSA paragraph: the core
// attention is followed by a grouped output projection to keep its cost down.
// Form implemented: the H query heads fall into G consecutive groups of H/G
// heads; group j's head outputs, concatenated (K = (H/G) d values per token),
// are multiplied by the group's own matrix W_j [K x dg]:
//   y[t, j*dg + n] = sum_k o[t, j*(H/G)*d + k] * W_j[k, n].
// Every group is a plain GEMM, so this is a batched GEMM on the MFMA units.
//
// Mapping (MI355X, wave64, MFMA 32x32x16 bf16 / 32x32x2 fp32): a workgroup
// computes a BM x BN = 128 x 128 tile of one group's output; its 4 waves each
// own a 64 x 64 quarter (2 x 2 MFMA tiles).  The K dimension is walked in
// 128-byte slices (64 bf16 / 32 fp32): A rows (tokens) are staged row-major
// in LDS, W is staged transposed (n-major, k contiguous) so that both MFMA
// operands are read as 16-byte k-runs.  The next slice is loaded into
// registers while the current one is multiplied.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

static constexpr int PJ_BM = 128;
static constexpr int PJ_BN = 128;
static constexpr int PJ_NT = 256;

// Position of the 4-k block kb in row n of the transposed W tile, XOR-swizzled
// by the row's 8-row group (spreads the 8-byte staging stores over the banks).
__device__ __forceinline__ int wt_block(int n, int kb, int nkb) { return kb ^ ((n >> 3) & (nkb - 1)); }

template <typename T>
__global__ __launch_bounds__(PJ_NT) void proj_kernel(ProjArgs a) {
  constexpr int VEC = 16 / sizeof(T);                 // elements per 16 bytes
  constexpr int BK = 8 * VEC;                         // k per slice: 128 bytes of a row
  constexpr int AS = BK + VEC;                        // A row stride in LDS (one 16-byte pad)
  constexpr int WS = BK;                              // W^T row stride (swizzled instead)
  constexpr int NKB = BK / 4;                         // 4-k blocks per W^T row
  constexpr int KSTEP = 16;                           // k per MFMA step (8 per lane half)
  constexpr int A_LD = PJ_BM * (BK / VEC) / PJ_NT;    // 16-byte A chunks per thread
  constexpr int W_TASKS = (BK / 4) * (PJ_BN / VEC);   // (4 k-rows x VEC n) tasks
  constexpr int W_LD = W_TASKS / PJ_NT;               // tasks per thread
  static_assert(A_LD * PJ_NT == PJ_BM * (BK / VEC) && W_LD * PJ_NT == W_TASKS, "tile split");

  __shared__ __align__(16) T As[PJ_BM * AS];
  __shared__ __align__(16) T Wt[PJ_BN * WS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;            // this wave's 64 x 64 quarter
  const int half = lane >> 5, col = lane & 31;
  const int m0 = blockIdx.x * PJ_BM, n0 = blockIdx.y * PJ_BN, g = blockIdx.z;
  const int K = a.K, ldo = a.G * a.K, ldy = a.G * a.dg;
  const T* o = reinterpret_cast<const T*>(a.o) + (size_t)g * K;
  const T* w = reinterpret_cast<const T*>(a.w) + (size_t)g * K * a.dg;
  T* y = reinterpret_cast<T*>(a.y) + (size_t)g * a.dg;

  // A rows past T read as zeros (their outputs are not stored)
  constexpr uint32_t OOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(o), (short)0, (int)min((size_t)0x7FFFFFFF, ((size_t)a.T * ldo) * sizeof(T)), 0x00020000);

  u32x4 areg[A_LD], wreg[W_LD][4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int c = tid + i * PJ_NT, r = c / (BK / VEC), ch = c % (BK / VEC);
      const int row = m0 + r;
      const uint32_t off = row < a.T ? (uint32_t)(((size_t)row * ldo + k0 + ch * VEC) * sizeof(T)) : OOB;
      areg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < W_LD; ++i) {
      const int c = tid + i * PJ_NT, kb = c / (PJ_BN / VEC), nc = c % (PJ_BN / VEC);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        wreg[i][u] = *reinterpret_cast<const u32x4*>(w + (size_t)(k0 + kb * 4 + u) * a.dg + n0 + nc * VEC);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int c = tid + i * PJ_NT, r = c / (BK / VEC), ch = c % (BK / VEC);
      *reinterpret_cast<u32x4*>(As + r * AS + ch * VEC) = areg[i];
    }
#pragma unroll
    for (int i = 0; i < W_LD; ++i) {
      const int c = tid + i * PJ_NT, kb = c / (PJ_BN / VEC), nc = c % (PJ_BN / VEC);
      const T* rows = reinterpret_cast<const T*>(wreg[i]);           // [4 k][VEC n]
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int n = nc * VEC + e;
        T four[4] = {rows[e], rows[VEC + e], rows[2 * VEC + e], rows[3 * VEC + e]};
        T* dst = Wt + n * WS + wt_block(n, kb, NKB) * 4;
        if constexpr (sizeof(T) == 2) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<uint2*>(four);
        else *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<u32x4*>(four);
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    store();
    __syncthreads();
    if (k0 + BK < K) load(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / KSTEP; ++ks) {
      Frag<T> af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        frag_load(af[i], As + (wm * 64 + i * 32 + col) * AS + ks * KSTEP + 8 * half);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = wn * 64 + j * 32 + col;
        const int kb = (ks * KSTEP + 8 * half) / 4;                  // two 4-k blocks
        const T* row = Wt + n * WS;
        if constexpr (sizeof(T) == 2) {
          const uint2 lo = *reinterpret_cast<const uint2*>(row + wt_block(n, kb, NKB) * 4);
          const uint2 hi = *reinterpret_cast<const uint2*>(row + wt_block(n, kb + 1, NKB) * 4);
          bfr[j].v = u32x4{lo.x, lo.y, hi.x, hi.y};
        } else {
          const f32x4 lo = *reinterpret_cast<const f32x4*>(row + wt_block(n, kb, NKB) * 4);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(row + wt_block(n, kb + 1, NKB) * 4);
          float* fv = reinterpret_cast<float*>(&bfr[j]);
          fv[0] = lo[0]; fv[1] = lo[1]; fv[2] = lo[2]; fv[3] = lo[3];
          fv[4] = hi[0]; fv[5] = hi[1]; fv[6] = hi[2]; fv[7] = hi[3];
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma32(acc[i][j], bfr[j], af[i]);   // C^T tile: rows n, columns t
    }
    __syncthreads();
  }

  // acc[i][j] holds the 32 x 32 block (n = wn*64 + j*32 + .., t = wm*64 + i*32 + ..)
  // in the C layout: lane (col = t, half) owns n rows 8q + 4 half + r.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = m0 + wm * 64 + i * 32 + col;
    if (t >= a.T) continue;
    T* yr = y + (size_t)t * ldy + n0 + wn * 64;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        T v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = from_f32<T>(acc[i][j][4 * q + r]);
        T* dst = yr + j * 32 + 8 * q + 4 * half;
        if constexpr (sizeof(T) == 2) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<uint2*>(v4);
        else *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<u32x4*>(v4);
      }
  }
}

hipError_t launch_proj(const ProjArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  dim3 grid((a.T + PJ_BM - 1) / PJ_BM, a.dg / PJ_BN, a.G);
  ProfScope ps("out_proj", st);
  if (a.f32) hipLaunchKernelGGL(proj_kernel<float>, grid, dim3(PJ_NT), 0, st, a);
  else hipLaunchKernelGGL(proj_kernel<bf16>, grid, dim3(PJ_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa
