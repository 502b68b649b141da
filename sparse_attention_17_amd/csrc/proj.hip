// Grouped output projection after the core attention.
// Method: DeepSeek-V4 summary (hyper.ai), "Method", CSA paragraph: the core
// attention is followed by a grouped output projection to keep its cost down.
// Form implemented: the H query heads fall into G consecutive groups of H/G
// heads; group j's head outputs, concatenated (K = (H/G) d values per token),
// are multiplied by the group's own matrix W_j, stored one row per output
// ([dg x K], as a linear layer's weight):
//   y[t, j*dg + n] = sum_k o[t, j*(H/G)*d + k] * W_j[n, k].
// Every group is a plain GEMM, so this is a batched GEMM on the MFMA units.
// Both operands are k-contiguous in memory, which is what an MFMA fragment
// holds (8 consecutive k per lane), so no transposition is needed anywhere.
//
// Mapping (MI355X, wave64, MFMA 32x32x16 bf16 / 32x32x2 fp32):
//   * many tokens: a workgroup computes a 128 x 128 tile of one group's
//     output; its 4 waves each own a 64 x 64 quarter (2 x 2 MFMA tiles).  K
//     is walked in 128-byte slices staged in LDS (rows padded by 16 bytes);
//     the next slice is loaded into registers while the current one is
//     multiplied.
//   * few tokens (decode): the weights dominate the traffic, so a workgroup
//     takes a 32 x 32 tile and its 4 waves split K four ways, reading their
//     fragments straight from memory; the four partial tiles are summed in
//     LDS.  The grid then has dg/32 x G workgroups per 32 tokens.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

static constexpr int PJ_BM = 128;
static constexpr int PJ_BN = 128;
static constexpr int PJ_NT = 256;
static constexpr int PJ_SKINNY_T = 32;      // token counts up to this use the split-K kernel

template <typename T>
__global__ __launch_bounds__(PJ_NT) void proj_kernel(ProjArgs a) {
  constexpr int VEC = 16 / sizeof(T);                 // elements per 16 bytes
  constexpr int BK = 8 * VEC;                         // k per slice: 128 bytes of a row
  constexpr int RS = BK + VEC;                        // LDS row stride (one 16-byte pad)
  constexpr int KSTEP = 16;                           // k per MFMA step (8 per lane half)
  constexpr int LD = PJ_BM * (BK / VEC) / PJ_NT;      // 16-byte chunks per thread per operand
  static_assert(LD * PJ_NT == PJ_BM * (BK / VEC) && PJ_BM == PJ_BN, "tile split");

  __shared__ __align__(16) T As[PJ_BM * RS];
  __shared__ __align__(16) T Ws[PJ_BN * RS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;            // this wave's 64 x 64 quarter
  const int half = lane >> 5, col = lane & 31;
  const int m0 = blockIdx.x * PJ_BM, n0 = blockIdx.y * PJ_BN, g = blockIdx.z;
  const int K = a.K, ldo = a.G * a.K, ldy = a.G * a.dg;
  const T* o = reinterpret_cast<const T*>(a.o) + (size_t)g * K;
  const T* w = reinterpret_cast<const T*>(a.w) + ((size_t)g * a.dg + n0) * K;
  T* y = reinterpret_cast<T*>(a.y) + (size_t)g * a.dg;

  // A rows past T read as zeros (their outputs are not stored)
  constexpr uint32_t OOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(o), (short)0, (int)min((size_t)0x7FFFFFFF, ((size_t)a.T * ldo) * sizeof(T)), 0x00020000);

  u32x4 areg[LD], wreg[LD];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int c = tid + i * PJ_NT, r = c / (BK / VEC), ch = c % (BK / VEC);
      const int row = m0 + r;
      const uint32_t off = row < a.T ? (uint32_t)(((size_t)row * ldo + k0 + ch * VEC) * sizeof(T)) : OOB;
      areg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
      wreg[i] = *reinterpret_cast<const u32x4*>(w + (size_t)r * K + k0 + ch * VEC);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int c = tid + i * PJ_NT, r = c / (BK / VEC), ch = c % (BK / VEC);
      *reinterpret_cast<u32x4*>(As + r * RS + ch * VEC) = areg[i];
      *reinterpret_cast<u32x4*>(Ws + r * RS + ch * VEC) = wreg[i];
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
      for (int i = 0; i < 2; ++i) frag_load(af[i], As + (wm * 64 + i * 32 + col) * RS + ks * KSTEP + 8 * half);
#pragma unroll
      for (int j = 0; j < 2; ++j) frag_load(bfr[j], Ws + (wn * 64 + j * 32 + col) * RS + ks * KSTEP + 8 * half);
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

// Few tokens: workgroup = 32 tokens x 32 outputs of one group; wave `wave`
// reduces k in [wave*K/4, (wave+1)*K/4), UNR MFMA steps per round of loads.
template <typename T>
__global__ __launch_bounds__(PJ_NT) void proj_skinny_kernel(ProjArgs a) {
  constexpr int KSTEP = 16;
  constexpr int UNR = 4;
  __shared__ float red[3][64][17];                    // waves 1..3 hand their tiles to wave 0

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 32, g = blockIdx.z;
  const int K = a.K, ldo = a.G * a.K, ldy = a.G * a.dg;
  const int kq = K / 4, kb = wave * kq;               // K is a multiple of 64: kq of 16
  const T* o = reinterpret_cast<const T*>(a.o) + (size_t)g * K;
  const T* wr = reinterpret_cast<const T*>(a.w) + ((size_t)g * a.dg + n0 + col) * K + kb + 8 * half;
  const int t = m0 + col;
  constexpr uint32_t OOB = 0x80000000u;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(o), (short)0, (int)min((size_t)0x7FFFFFFF, ((size_t)a.T * ldo) * sizeof(T)), 0x00020000);
  const uint32_t obase = t < a.T ? (uint32_t)(((size_t)t * ldo + kb + 8 * half) * sizeof(T)) : OOB;

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  auto ofrag = [&](Frag<T>& f, int k) {
    const uint32_t off = obase == OOB ? OOB : obase + (uint32_t)(k * sizeof(T));
    if constexpr (sizeof(T) == 2) {
      f.v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
    } else {
      const f32x4 lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
      const f32x4 hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off == OOB ? OOB : off + 16, 0, 0));
      for (int i = 0; i < 4; ++i) { f.v[i] = lo[i]; f.v[4 + i] = hi[i]; }
    }
  };
  for (int k = 0; k < kq; k += KSTEP * UNR) {
    Frag<T> af[UNR], bfr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kk = min(k + u * KSTEP, kq - KSTEP);  // clamped: repeats are not accumulated
      ofrag(af[u], kk);
      frag_load(bfr[u], wr + kk);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (k + u * KSTEP < kq) mma32(acc, bfr[u], af[u]);
  }
  if (wave > 0)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave - 1][lane][r] = acc[r];
  __syncthreads();
  if (wave > 0 || t >= a.T) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] += red[0][lane][r] + red[1][lane][r] + red[2][lane][r];
  T* yr = reinterpret_cast<T*>(a.y) + (size_t)t * ldy + (size_t)g * a.dg + n0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    T v4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v4[r] = from_f32<T>(acc[4 * q + r]);
    T* dst = yr + 8 * q + 4 * half;
    if constexpr (sizeof(T) == 2) *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<uint2*>(v4);
    else *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<u32x4*>(v4);
  }
}

hipError_t launch_proj(const ProjArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  ProfScope ps("out_proj", st);
  if (a.T <= PJ_SKINNY_T) {
    dim3 grid(1, a.dg / 32, a.G);
    if (a.f32) hipLaunchKernelGGL(proj_skinny_kernel<float>, grid, dim3(PJ_NT), 0, st, a);
    else hipLaunchKernelGGL(proj_skinny_kernel<bf16>, grid, dim3(PJ_NT), 0, st, a);
  } else {
    dim3 grid((a.T + PJ_BM - 1) / PJ_BM, a.dg / PJ_BN, a.G);
    if (a.f32) hipLaunchKernelGGL(proj_kernel<float>, grid, dim3(PJ_NT), 0, st, a);
    else hipLaunchKernelGGL(proj_kernel<bf16>, grid, dim3(PJ_NT), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace csa
