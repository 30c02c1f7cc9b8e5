// conv1d.hip -- causal depthwise convolution ahead of the scan, for gfx950.
//
// The width-K (d_conv, 4 in Mamba) causal 1-D convolution that mixes each
// token with the K-1 before it before the selective SSM (section 3.3 of the
// "Understanding Mamba and Selective State Space Models (SSMs)" blog; the
// causal-conv1d layer named in the Mamba README):
//
//   out[b,d,t] = act( bias[d] + sum_{k<K} w[d,k] x[b,d,t-(K-1)+k] ),   x[t<0] = 0
//
// act = silu or identity.  A pure stream over x: each thread produces eight
// consecutive tokens of one row from one 16-byte (bf16) or two (fp32) loads
// of its own tokens plus the previous eight tokens for the K-1 halo (the
// neighbouring thread's data, served by the caches); rows whose tokens are
// not 16-byte aligned take a token-per-thread path.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

constexpr int kV = 8;   // tokens per thread

template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16lo(w[i]);
            v[2 * i + 1] = bf16hi(w[i]);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
        *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
    static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <> struct Vec<float> {
    static __device__ __forceinline__ void load(const float* p, float* v) {
        const float4 a = reinterpret_cast<const float4*>(p)[0];
        const float4 b = reinterpret_cast<const float4*>(p)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void store(float* p, const float* v) {
        reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
    static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};

__device__ __forceinline__ float act(float v, bool silu) { return silu ? silu_scaled(v, 1.0f) : v; }

constexpr int kConvThreads = 256;

// K <= 8: the halo fits in the previous eight tokens.  Each row gets whole
// workgroups (`bpr` of them), so the row and channel of a workgroup come
// from one scalar division instead of per-thread 64-bit ones.
template <typename Tin, typename Tout, int K, bool SILU>
__global__ __launch_bounds__(kConvThreads) void conv_vec_kernel(ConvArgs a, uint32_t bpr) {
    const int64_t groups = a.L / kV;
    const uint32_t blk = blockIdx.x;
    const int64_t row = blk / bpr;
    const int64_t g = (int64_t)(blk - (uint32_t)row * bpr) * kConvThreads + threadIdx.x;
    if (g >= groups) return;
    const int64_t d = row % a.dim;
    const Tin* x = reinterpret_cast<const Tin*>(a.x) + row * a.L + g * kV;
    float cur[kV], prev[kV];
    Vec<Tin>::load(x, cur);
    if (g > 0) {
        Vec<Tin>::load(x - kV, prev);
    } else {
#pragma unroll
        for (int i = 0; i < kV; ++i) prev[i] = 0.0f;
    }
    float w[K];
#pragma unroll
    for (int k = 0; k < K; ++k) w[k] = a.w[d * K + k];
    const float b0 = a.bias ? a.bias[d] : 0.0f;
    float o[kV];
#pragma unroll
    for (int i = 0; i < kV; ++i) {
        float acc = b0;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int s = i - (K - 1) + k;   // -7 .. 7
            acc = __builtin_fmaf(w[k], s >= 0 ? cur[s] : prev[s + kV], acc);
        }
        o[i] = act(acc, SILU);
    }
    Vec<Tout>::store(reinterpret_cast<Tout*>(a.out) + row * a.L + g * kV, o);
}

// Any K, any alignment: one token per thread.
template <typename Tin, typename Tout, bool SILU>
__global__ __launch_bounds__(256) void conv_tok_kernel(ConvArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= a.batch * a.dim * a.L) return;
    const int64_t row = gid / a.L;
    const int64_t t = gid - row * a.L;
    const int64_t d = row % a.dim;
    const Tin* x = reinterpret_cast<const Tin*>(a.x) + row * a.L;
    float acc = a.bias ? a.bias[d] : 0.0f;
    for (int k = 0; k < a.K; ++k) {
        const int64_t s = t - (a.K - 1) + k;
        if (s >= 0) acc = __builtin_fmaf(a.w[d * a.K + k], Vec<Tin>::ld(x, s), acc);
    }
    Vec<Tout>::st(reinterpret_cast<Tout*>(a.out) + row * a.L, t, act(acc, SILU));
}

template <typename Tin, typename Tout, bool SILU>
hipError_t launch_silu(const ConvArgs& a, hipStream_t stream) {
    KTime kt("conv1d", stream);
    const int64_t bpr = (a.L / kV + kConvThreads - 1) / kConvThreads;   // workgroups per row
    if (a.vec_ok && a.K >= 1 && a.K <= kV && a.batch * a.dim * bpr < 0x7fffffff) {
        const unsigned blocks = (unsigned)(a.batch * a.dim * bpr);
        switch (a.K) {
#define SELSCAN_CONV_K(KK)                                                                                          \
    case KK:                                                                                                        \
        hipLaunchKernelGGL((conv_vec_kernel<Tin, Tout, KK, SILU>), dim3(blocks), dim3(kConvThreads), 0, stream, a, \
                           (uint32_t)bpr);                                                                          \
        break;
            SELSCAN_CONV_K(1) SELSCAN_CONV_K(2) SELSCAN_CONV_K(3) SELSCAN_CONV_K(4)
            SELSCAN_CONV_K(5) SELSCAN_CONV_K(6) SELSCAN_CONV_K(7) SELSCAN_CONV_K(8)
#undef SELSCAN_CONV_K
        }
    } else {
        const int64_t threads = a.batch * a.dim * a.L;
        hipLaunchKernelGGL((conv_tok_kernel<Tin, Tout, SILU>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_dt(const ConvArgs& a, hipStream_t stream) {
    return a.silu ? launch_silu<Tin, Tout, true>(a, stream) : launch_silu<Tin, Tout, false>(a, stream);
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs& a, int in_bf16, int out_bf16, hipStream_t stream) {
    if (in_bf16 && out_bf16) return launch_dt<uint16_t, uint16_t>(a, stream);
    if (in_bf16) return launch_dt<uint16_t, float>(a, stream);
    if (out_bf16) return launch_dt<float, uint16_t>(a, stream);
    return launch_dt<float, float>(a, stream);
}

}  // namespace selscan
