// SwiGLU elementwise math shared by the SwiGLU kernels and the MX quantizer
// that fuses it: one definition, so every kernel computes the same bits.
// silu(g) * up in fp32 with a sigmoid whose exponential never overflows, and
// the product rule for the backward, each result rounded once to bf16
// (nearest even).  [P4 "MoE" (the expert MLP between the two grouped GEMMs).]
#pragma once

#include "device_common.hpp"

namespace fp8moe {

typedef float sw_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 sw_bf16x2 __attribute__((ext_vector_type(2)));

// sigmoid(g) in fp32, in the form whose exponential never overflows:
// 1 / (1 + e^-g) for g >= 0 and e^g / (1 + e^g) below, both from the one
// exponential e^-|g| (a wave whose lanes take both signs evaluates it once).
// The denominator lies in [1, 2], so the hardware reciprocal (1 ulp) times the
// numerator stands in for the division (within 2 ulp; the kernels that use it
// are bound by their arithmetic, and the division's exact-rounding sequence
// was a fifth of it).
__device__ __forceinline__ float sw_sigmoid(float g) {
  const float e = expf(-fabsf(g));
  return (g >= 0.0f ? 1.0f : e) * __builtin_amdgcn_rcpf(1.0f + e);
}

// Two fp32 values -> one word of two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t sw_pack(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(sw_f32x2{a, b}, sw_bf16x2));
}

// A2 chunk (8 columns) from the gate and up chunks.
__device__ __forceinline__ u32x4 sw_fwd_chunk(const u32x4& g, const u32x4& u) {
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float g0 = bf16_lo(gw[k]), g1 = bf16_hi(gw[k]);
    const float u0 = bf16_lo(uw[k]), u1 = bf16_hi(uw[k]);
    o[k] = sw_pack(g0 * sw_sigmoid(g0) * u0, g1 * sw_sigmoid(g1) * u1);
  }
  return u32x4{o[0], o[1], o[2], o[3]};
}

// dH1 chunks (gate part, up part; 8 columns each) from dA2, gate and up chunks.
__device__ __forceinline__ void sw_bwd_chunk(const u32x4& d, const u32x4& g, const u32x4& u, u32x4& dg, u32x4& du) {
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w}, gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t og[4], ou[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float rg[2], ru[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float dv = h ? bf16_hi(dw[k]) : bf16_lo(dw[k]);
      const float gv = h ? bf16_hi(gw[k]) : bf16_lo(gw[k]);
      const float uv = h ? bf16_hi(uw[k]) : bf16_lo(uw[k]);
      const float s = sw_sigmoid(gv);
      rg[h] = dv * uv * s * (1.0f + gv * (1.0f - s));
      ru[h] = dv * gv * s;
    }
    og[k] = sw_pack(rg[0], rg[1]);
    ou[k] = sw_pack(ru[0], ru[1]);
  }
  dg = u32x4{og[0], og[1], og[2], og[3]};
  du = u32x4{ou[0], ou[1], ou[2], ou[3]};
}

}  // namespace fp8moe
