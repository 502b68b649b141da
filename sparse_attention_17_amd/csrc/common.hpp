// Device helpers shared by the gfx950 kernels: element types, bf16 rounding,
// MFMA fragment wrappers, wave/block reductions and scans.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

struct bf16 { uint16_t x; };   // storage type: raw bfloat16 bits

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float((uint32_t)v.x << 16); }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two values in one v_cvt_pk_bf16_f32 (the same rounding as two scalar
// conversions): lo in bits 0..15, hi in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float f) { bf16 r; r.x = (uint16_t)f32_to_bf16_bits(f); return r; }

// ---------------------------------------------------------------------------
// MFMA fragments.  A "k-chunk fragment" is the 8 consecutive k-values one lane
// contributes to one bf16 MFMA (16x16x32 or 32x32x16).  For fp32 data the
// same 8 k-values are fed to 8 fp32 MFMAs (16x16x4 / 32x32x2) in which the
// lane's single k-slot stands for k = 8*(lane group) + s at step s, so both
// element types share one fragment layout and one reduction order per lane.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;

// Workgroups of a 1-D launch are dealt to the chip's 8 XCDs round-robin
// (workgroup i to XCD i mod 8), each XCD with its own L2.  xcd_rows maps
// workgroup `bid` of a launch of rows x per_row workgroups to (row, j) so
// that, when rows is a multiple of 8, every workgroup of one row runs on the
// XCD of that row (row mod 8): what one kernel writes for a row then stays in
// the L2 that the next kernel's workgroups for the row read.  Other row counts
// keep row-major order.
struct RowJ { int row, j; };
__device__ __forceinline__ RowJ xcd_rows(int bid, int rows, int per_row) {
  if ((rows & 7) == 0) {
    const int q = bid >> 3, nb8 = rows >> 3;
    return RowJ{(bid & 7) + 8 * (q % nb8), q / nb8};
  }
  return RowJ{bid / per_row, bid % per_row};
}
template <> struct Frag<bf16> { u32x4 v; };          // 8 packed bf16
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void frag_load(Frag<bf16>& f, const void* p) {
  f.v = *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void frag_load(Frag<float>& f, const void* p) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p);
  f32x4 a = q[0], b = q[1];
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}
__device__ __forceinline__ void frag_zero(Frag<bf16>& f) { f.v = u32x4{0, 0, 0, 0}; }
__device__ __forceinline__ void frag_zero(Frag<float>& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = 0.f;
}
// Build a fragment from 8 fp32 values (bf16: round to nearest even).
__device__ __forceinline__ void frag_from_f32(Frag<bf16>& f, const float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
}
__device__ __forceinline__ void frag_from_f32(Frag<float>& f, const float* x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = x[i];
}

// C(32x32) += A(32 x 16) * B(16 x 32)
__device__ __forceinline__ void mma32(f32x16& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                              __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[s], b.v[s], c, 0, 0, 0);
}
// C(16x16) += A(16 x 32) * B(32 x 16)
__device__ __forceinline__ void mma16(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                              __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Reductions / scans.
// ---------------------------------------------------------------------------
// Wave-wide scans and reductions move lanes with DPP (VALU operand
// modifiers, no LDS round trip).  GFX9 controls: row_shr:n (0x110 + n) inside
// each 16-lane row, row_bcast:15 (0x142: lane 15 of a row to the next row)
// and row_bcast:31 (0x143: lane 31 to rows 2 and 3).  Lanes with no source,
// and rows outside ROW_MASK, receive `id`.  Callers run them with every lane
// of the wave active.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t id, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROW_MASK, 0xf, false);
}
// Inclusive scan of the associative `op` (identity `id`) over the 64 lanes:
// shifts by 1, 2, 4, 8 inside the rows, then the row totals carried up.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp_move<0x111, 0xf>(id, v));
  v = op(v, dpp_move<0x112, 0xf>(id, v));
  v = op(v, dpp_move<0x114, 0xf>(id, v));
  v = op(v, dpp_move<0x118, 0xf>(id, v));
  v = op(v, dpp_move<0x142, 0xa>(id, v));
  v = op(v, dpp_move<0x143, 0xc>(id, v));
  return v;
}
// Reduction of `op` over the wave: the scan's last lane, read as a scalar.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, uint32_t id, Op op) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(v, id, op), 63);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_reduce(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce(__float_as_uint(v), 0xFF800000u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_reduce(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  return wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
// Exclusive prefix sum over a block of NT threads; `smem` holds NT/64 words.
// Returns the exclusive prefix; *total receives the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* smem, uint32_t* total) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan(v);
  if (lane == 63) smem[wv] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    uint32_t s = smem[i];
    if (i < wv) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

}  // namespace csa
