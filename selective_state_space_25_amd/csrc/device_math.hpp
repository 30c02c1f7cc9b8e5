// device_math.hpp -- per-token scalar math of the selective scan on gfx950.
//
// Everything is fp32 and built from the hardware's base-2 transcendental
// instructions (v_exp_f32, v_log_f32, v_rcp_f32), which on gfx950 issue at
// half the FMA rate.  The functions work in log2 units so that no extra
// ln2/log2e scaling is needed on the per-update path:
//
//   w = softplus(v) / ln2 = log2(1 + 2^(v log2 e))      ("Delta in log2 units")
//   exp(Delta * A)       = 2^(w * A)
//
// softplus keeps Delta positive (tip at the end of section 2.2 of the
// "Understanding Mamba and Selective State Space Models (SSMs)" blog).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace selscan {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInvLn2 = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// bfloat16 <-> fp32.  Widening is exact (the bf16 bits are the upper half of
// the fp32 word); narrowing rounds to nearest even in one instruction
// (v_cvt_pk_bf16_f32) through the compiler's bfloat conversion.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    f32x2_t v = {lo, hi};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

// log2(1 + 2^vl) for any vl, accurate to a few ulp relative everywhere.
// Written as max(vl, 0) + log2(1 + e) with e = 2^-|vl| in (0, 1]; the
// rounding error of 1 + e is recovered exactly (Fast2Sum, since 1 >= e) and
// added back to first order, which keeps the tiny-Delta regime (e << 1,
// where log2(1 + e) ~ e log2 e) accurate instead of losing it to the rounding
// of 1 + e.
__device__ __forceinline__ float softplus_log2(float vl) {
    float e = fast_exp2(-fabsf(vl));
    float s = 1.0f + e;
    float err = e - (s - 1.0f);
    float l = fast_log2(s);
    return fmaxf(vl, 0.0f) + __builtin_fmaf(err, kLog2e, l);
}

// silu(z) * scale = scale * z / (1 + e^-z); the scale folds in a constant at
// no cost (the divisor is formed as (1 + t) / scale by one FMA).
__device__ __forceinline__ float silu_scaled(float z, float inv_scale) {
    float t = fast_exp2(-z * kLog2e);
    float d = __builtin_fmaf(t, inv_scale, inv_scale);
    return z * fast_rcp(d);
}

}  // namespace selscan
