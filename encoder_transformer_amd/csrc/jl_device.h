// Device helpers shared by the kernel translation units of libjl (gfx950).
#pragma once

#include "jl_internal.h"

#include <math.h>

namespace jl {
namespace dev {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// fragments and matrix-core steps
// ---------------------------------------------------------------------------

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ inline Frag<bf16> load_frag(const bf16 *p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8 *>(p);
  return f;
}
__device__ inline Frag<float> load_frag(const float *p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4 *>(p);
  f.hi = *reinterpret_cast<const f32x4 *>(p + 4);
  return f;
}
__device__ inline void store_frag(bf16 *p, const Frag<bf16> &f) {
  *reinterpret_cast<bf16x8 *>(p) = f.v;
}
__device__ inline void store_frag(float *p, const Frag<float> &f) {
  *reinterpret_cast<f32x4 *>(p) = f.lo;
  *reinterpret_cast<f32x4 *>(p + 4) = f.hi;
}
__device__ inline float frag_get(const Frag<bf16> &f, int e) { return (float)f.v[e]; }
__device__ inline float frag_get(const Frag<float> &f, int e) { return e < 4 ? f.lo[e] : f.hi[e - 4]; }

// Build a fragment from 8 FP32 values (bf16: round to nearest even).
__device__ inline void frag_from(Frag<bf16> &f, const float *v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)v[e];
}
__device__ inline void frag_from(Frag<float> &f, const float *v) {
  f.lo = f32x4{v[0], v[1], v[2], v[3]};
  f.hi = f32x4{v[4], v[5], v[6], v[7]};
}

// acc[16x16] += A(16 x 32) . B(32 x 16); lane (i + 16g) supplies A row i and
// B column i at k = 8g .. 8g+7.
__device__ inline void mfma(f32x4 &acc, const Frag<bf16> &a, const Frag<bf16> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ inline void mfma(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], acc, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], acc, 0, 0, 0);
}

template <typename T> __device__ inline T to_elem(float v);
template <> __device__ inline bf16 to_elem<bf16>(float v) { return (bf16)v; }
template <> __device__ inline float to_elem<float>(float v) { return v; }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over each 16-lane row of the wave without LDS: butterflies by DPP (xor
// 1 and xor 2 through quad permutes, then the 8- and 16-lane mirrors).  Every
// lane of a row gets the same value and the summation order is fixed, so any
// kernel using it reduces a row of data bit-identically.
__device__ inline float row16_sum(float v) {
#pragma clang fp contract(off)
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror (8 lanes)
  v += dpp<0x140>(v);  // row_mirror (16 lanes)
  return v;
}

// LayerNorm statistics of one 384-wide row held by a 16-lane row of the
// wave: lane j holds columns 64 c + 4 j .. 64 c + 4 j + 3 in x[c], c = 0..5.
// Two passes, biased variance.  Shared by the LayerNorm kernel and the fused
// LayerNorm of the GEMM, which therefore produce identical operands.
__device__ inline void ln_row16(const f32x4 (&x)[6], float &mean, float &rstd) {
#pragma clang fp contract(off)
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 6; ++c) s += (x[c][0] + x[c][1]) + (x[c][2] + x[c][3]);
  mean = row16_sum(s) * (1.0f / kWidth);
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < 6; ++c) {
    const float d0 = x[c][0] - mean, d1 = x[c][1] - mean, d2 = x[c][2] - mean, d3 = x[c][3] - mean;
    q += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
  }
  rstd = rsqrtf(row16_sum(q) * (1.0f / kWidth) + kLnEps);
}

// Maximum over each 16-lane row of the wave (same butterflies as row16_sum).
__device__ inline float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// The same GELU with erf from Abramowitz & Stegun 7.1.26 (|error| <= 1.5e-7):
// for x >= 0, erfc(x) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
// t = 1 / (1 + p x).  With x = |z| / sqrt(2) and h = z erfc(x) / 2,
// gelu(z) = z Phi(z) is z - h for z >= 0 and h for z < 0.  In FP32 the
// result is within 3.4e-7 of the exact GELU on [-12, 12]; used where the
// output is rounded to bf16.
__device__ inline float gelu_erf_fast(float z) {
  const float x = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  float q = fmaf(1.061405429f, t, -1.453152027f);
  q = fmaf(q, t, 1.421413741f);
  q = fmaf(q, t, -0.284496736f);
  q = fmaf(q, t, 0.254829592f);
  q = q * t;
  const float e = __builtin_amdgcn_exp2f(x * x * -1.4426950408889634f);
  const float h = 0.5f * z * (q * e);
  return z >= 0.f ? z - h : h;
}

}  // namespace dev
}  // namespace jl
