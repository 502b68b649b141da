// Block compressor: softmax-gated pooling of every m-token block of K, V and
// the indexer keys into one entry (CSA with m, HCA with m').
// Method: DeepSeek-V4 summary (hyper.ai), "Method", CSA paragraph — m tokens
// become one entry through learnable compression weights and positional
// biases; HCA paragraph — m' tokens with no overlap between entries, which
// the page states for HCA only.  Form implemented, for entry j and a window of `width`
// tokens ending where block j ends (width = m: the block itself; width > m:
// windows of consecutive entries overlap by width - m tokens):
//   rows t = (j+1)m - width + i, i = 0..width-1, t >= 0 (earlier ones absent)
//   a_i = k_t . g + b_i,  p = softmax over the window's rows,
//   Kc = sum p_i k_t,  Vc = sum p_i v_t,  KIc = sum p_i kI_t.
//
// Mapping: one wavefront per block.  A row of d elements is read by G lanes
// with 16-byte loads (G = d*sizeof(T)/16), so a wave covers R = 64/G rows per
// step and streams the block once with an online softmax per row slot; the R
// slot states are merged with cross-lane shuffles at the end.  HBM-bound:
// each input byte is read exactly once, each output byte written once.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

template <typename T, int D, int DI>
__global__ __launch_bounds__(256) void compress_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ ki,
    const float* __restrict__ gate, const float* __restrict__ pos_bias,
    int T_len, int m, int width, int Nc, int Nc_cap,
    T* __restrict__ kc, T* __restrict__ vc, T* __restrict__ kic) {
  constexpr int VEC = 16 / sizeof(T);          // elements per lane per K/V row
  constexpr int G = D / VEC;                   // lanes per row
  constexpr int R = 64 / G;                    // rows per wave step
  constexpr int KIV = DI / G;                  // indexer-key elements per lane
  constexpr int U = 4;                         // row steps in flight
  static_assert(G >= 1 && G <= 64 && KIV >= 1, "unsupported shape");

  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (j >= Nc) return;
  const int slot = lane / G, col = lane % G;

  float g[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) g[e] = gate[col * VEC + e];

  float M = -INFINITY, S = 0.f;
  float ak[VEC], av[VEC], ai[KIV];
#pragma unroll
  for (int e = 0; e < VEC; ++e) { ak[e] = 0.f; av[e] = 0.f; }
#pragma unroll
  for (int e = 0; e < KIV; ++e) ai[e] = 0.f;

  // window rows t = t0 + i; rows before the sequence start are absent
  const long long t0 = (long long)(j + 1) * m - width;
  const int i_lo = t0 < 0 ? (int)-t0 : 0;
  const size_t seq0 = (size_t)b * T_len;
  const bool has_ki = (ki != nullptr);

  for (int i0 = i_lo; i0 < width; i0 += R * U) {
    T rk[U][VEC], rv[U][VEC], ri[U][KIV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * R + slot;
      if (i < width) {
        const size_t r = seq0 + (size_t)(t0 + i);
#pragma unroll
        for (int e = 0; e < VEC; e += 16 / sizeof(T)) {
          *reinterpret_cast<u32x4*>(&rk[u][e]) =
              *reinterpret_cast<const u32x4*>(k + r * D + col * VEC + e);
          *reinterpret_cast<u32x4*>(&rv[u][e]) =
              *reinterpret_cast<const u32x4*>(v + r * D + col * VEC + e);
        }
        if (has_ki) {
#pragma unroll
          for (int e = 0; e < KIV; ++e) ri[u][e] = ki[r * DI + col * KIV + e];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * R + slot;
      // gate logit: partial dot over this lane's columns, reduced over G lanes
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) a = fmaf(to_f32(rk[u][e]), g[e], a);
#pragma unroll
      for (int o = 1; o < G; o <<= 1) a += __shfl_xor(a, o, 64);
      if (i < width) {
        if (pos_bias) a += pos_bias[i];
        const float Mn = fmaxf(M, a);
        const float c = __expf(M - Mn);
        const float p = __expf(a - Mn);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          ak[e] = fmaf(ak[e], c, p * to_f32(rk[u][e]));
          av[e] = fmaf(av[e], c, p * to_f32(rv[u][e]));
        }
        if (has_ki) {
#pragma unroll
          for (int e = 0; e < KIV; ++e) ai[e] = fmaf(ai[e], c, p * to_f32(ri[u][e]));
        }
        S = fmaf(S, c, p);
        M = Mn;
      }
    }
  }

  // merge the R row-slot states (slots hold disjoint rows of the block)
#pragma unroll
  for (int o = G; o < 64; o <<= 1) {
    const float M2 = __shfl_xor(M, o, 64);
    const float S2 = __shfl_xor(S, o, 64);
    const float Mn = fmaxf(M, M2);
    const float c1 = (M == -INFINITY) ? 0.f : __expf(M - Mn);
    const float c2 = (M2 == -INFINITY) ? 0.f : __expf(M2 - Mn);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      ak[e] = ak[e] * c1 + __shfl_xor(ak[e], o, 64) * c2;
      av[e] = av[e] * c1 + __shfl_xor(av[e], o, 64) * c2;
    }
#pragma unroll
    for (int e = 0; e < KIV; ++e) ai[e] = ai[e] * c1 + __shfl_xor(ai[e], o, 64) * c2;
    S = S * c1 + S2 * c2;
    M = Mn;
  }

  if (slot == 0) {
    const float inv = 1.f / S;
    const size_t orow = (size_t)b * Nc_cap + j;
    T ok[VEC], ov[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      ok[e] = from_f32<T>(ak[e] * inv);
      ov[e] = from_f32<T>(av[e] * inv);
    }
    *reinterpret_cast<u32x4*>(kc + orow * D + col * VEC) = *reinterpret_cast<u32x4*>(ok);
    *reinterpret_cast<u32x4*>(vc + orow * D + col * VEC) = *reinterpret_cast<u32x4*>(ov);
    if (has_ki) {
#pragma unroll
      for (int e = 0; e < KIV; ++e) kic[orow * DI + col * KIV + e] = from_f32<T>(ai[e] * inv);
    }
  }
}

template <typename T, int D, int DI>
static hipError_t launch_t(const CompressArgs& a, hipStream_t st) {
  const int Nc = a.T / a.m;
  if (Nc == 0 || a.B == 0) return hipSuccess;
  dim3 grid((Nc + 3) / 4, a.B);
  ProfScope ps("compress", st);
  hipLaunchKernelGGL((compress_kernel<T, D, DI>), grid, dim3(256), 0, st,
                     (const T*)a.k, (const T*)a.v, (const T*)a.ki, a.gate, a.pos_bias,
                     a.T, a.m, a.width, Nc, a.Nc_cap, (T*)a.kc, (T*)a.vc, (T*)a.kic);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
  // dI only shapes the indexer-key part; when ki is absent any instance works.
  const int dI = a.ki ? a.dI : 32;
  if (a.f32) {
    if (a.d == 64 && dI == 32) return launch_t<float, 64, 32>(a, st);
    if (a.d == 64 && dI == 64) return launch_t<float, 64, 64>(a, st);
    if (a.d == 128 && dI == 32) return launch_t<float, 128, 32>(a, st);
    if (a.d == 128 && dI == 64) return launch_t<float, 128, 64>(a, st);
  } else {
    if (a.d == 64 && dI == 32) return launch_t<bf16, 64, 32>(a, st);
    if (a.d == 64 && dI == 64) return launch_t<bf16, 64, 64>(a, st);
    if (a.d == 128 && dI == 32) return launch_t<bf16, 128, 32>(a, st);
    if (a.d == 128 && dI == 64) return launch_t<bf16, 128, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace csa
