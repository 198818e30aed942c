// Device-side helpers shared by the gfx950 kernels of the action head:
// bf16 / e4m3 storage types, conversions, and wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gr00t {

// bf16 storage: the upper 16 bits of an IEEE binary32 value.
struct bf16 {
  uint16_t u;
};
// OCP E4M3 ("fn") storage: 1 sign, 4 exponent (bias 7), 3 mantissa bits.
struct fp8e4m3 {
  uint8_t u;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN payloads are not preserved).
// fp32 -> bf16, round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
typedef __bf16 bf16x2_n __attribute__((ext_vector_type(2)));
typedef float floatx2_n __attribute__((ext_vector_type(2)));
// two values -> packed bf16 pair (a in the low half), one instruction
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2_n){a, b}, bf16x2_n));
}

// e4m3 code -> bf16 bits (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ uint16_t e4m3_to_bf16(uint32_t c) {
  uint32_t s = (c & 0x80u) << 8;
  uint32_t e = (c >> 3) & 0xFu;
  uint32_t m = c & 0x7u;
  if (e != 0) return (uint16_t)(s | ((e + 120u) << 7) | (m << 4));
  // subnormal: m * 2^-9, m = 1..7 (m = 0 gives +-0)
  float v = (float)m * (1.0f / 512.0f);
  return (uint16_t)(s | (__float_as_uint(v) >> 16));
}

__device__ __forceinline__ float e4m3_to_f(uint32_t c) { return bf16_to_f(e4m3_to_bf16(c)); }

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld<bf16>(const bf16* p) { return bf16_to_f(p->u); }
template <>
__device__ __forceinline__ float ld<fp8e4m3>(const fp8e4m3* p) { return e4m3_to_f(p->u); }

template <typename T>
__device__ __forceinline__ void st(T* p, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st<bf16>(bf16* p, float v) { p->u = f_to_bf16(v); }

// Wave64 reductions in the pairing of the xor butterfly: lane i combines its value with
// that of lane i ^ 32, then i ^ 16, i ^ 8, i ^ 4, i ^ 2, i ^ 1. The stages run on the SIMD
// rather than through LDS: i ^ 32 and i ^ 16 with the gfx950 permlane swaps (a swap of a
// register with itself leaves, in every lane, the lane's own value in one result and its
// partner's in the other), i ^ 8 and i ^ 4 as rotations of each 16-lane row by 8 and by 4
// (once the values repeat with period 16, resp. 8, inside a row, the rotated-in value is the
// xor partner's), i ^ 2 and i ^ 1 as quad permutations. Every stage combines the same two
// operands as the butterfly, so the result is bitwise that of the butterfly, in every lane.
// All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {  // row_mask, bank_mask 0xF: every lane
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_ROW_ROR8 = 0x128, DPP_ROW_ROR4 = 0x124, DPP_QUAD_XOR2 = 0x4E, DPP_QUAD_XOR1 = 0xB1;

// own and partner value (in either order) for partner lane i ^ 32 (L32) or i ^ 16
template <bool L32>
__device__ __forceinline__ void xor_pair(float v, float& a, float& b) {
  const uint32_t u = __float_as_uint(v);
  if constexpr (L32) {
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
  } else {
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
  }
}

struct SumOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// stages i ^ 32 and i ^ 16 of N independent values, interleaved
template <int N, typename Op>
__device__ __forceinline__ void wave_reduce_rows(float (&v)[N], Op op) {
  float a[N], b[N];
#pragma unroll
  for (int j = 0; j < N; ++j) xor_pair<true>(v[j], a[j], b[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = op(a[j], b[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) xor_pair<false>(v[j], a[j], b[j]);
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = op(a[j], b[j]);
}
// stages i ^ 8 .. i ^ 1 (inside 16-lane rows) of N independent values, interleaved
template <int N, typename Op>
__device__ __forceinline__ void wave_reduce_in_row(float (&v)[N], Op op) {
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = op(v[j], dpp_f<DPP_ROW_ROR8>(v[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = op(v[j], dpp_f<DPP_ROW_ROR4>(v[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = op(v[j], dpp_f<DPP_QUAD_XOR2>(v[j]));
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = op(v[j], dpp_f<DPP_QUAD_XOR1>(v[j]));
}
// N independent wave sums (each bitwise the butterfly's), interleaved
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
  wave_reduce_rows(v, SumOp{});
  wave_reduce_in_row(v, SumOp{});
}
__device__ __forceinline__ float wave_sum(float v) {
  float a[1] = {v};
  wave_sum_n(a);
  return a[0];
}
__device__ __forceinline__ float wave_max(float v) {
  float a[1] = {v};
  wave_reduce_rows(a, MaxOp{});
  wave_reduce_in_row(a, MaxOp{});
  return a[0];
}
// the stages i ^ 16 then i ^ 32 alone (values that already agree inside each 16-lane row)
template <typename Op>
__device__ __forceinline__ float across_rows_16_32(float v, Op op) {
  float a, b;
  xor_pair<false>(v, a, b);
  v = op(a, b);
  xor_pair<true>(v, a, b);
  return op(a, b);
}
// sum over the 16-lane row (partners i ^ 8 .. i ^ 1), bitwise the butterfly's
__device__ __forceinline__ float row16_sum(float v) {
  float a[1] = {v};
  wave_reduce_in_row(a, SumOp{});
  return a[0];
}

// erf from Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26
// (|error| <= 1.5e-7): one reciprocal, one exponential and a degree-5 polynomial, with no
// branches, for the GELU in GEMM epilogues.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
  const float poly = t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  return copysignf(1.0f - poly * __expf(-ax * ax), x);
}
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erf_as(x * 0.70710678118654752f)); }
__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// Buffer-descriptor loads: an offset past the descriptor's byte range reads 0 (no fault,
// no branch), so every lane can issue the same loads.
typedef int int32x4_t __attribute__((ext_vector_type(4)));
constexpr int OOB = 0x7FFFFFF0;  // buffer offset that is always out of range (reads 0)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  int32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}
__device__ __forceinline__ uint8_t buf_load1(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

}  // namespace gr00t
