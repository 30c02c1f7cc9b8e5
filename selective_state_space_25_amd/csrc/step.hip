// step.hip -- one-token state update (decoding) for gfx950.
//
// The recurrent view of the selective SSM (blog "Understanding Mamba and
// Selective State Space Models (SSMs)" section 2.2, second cut; the
// streaming use of the step function on the tutorial and skill pages):
// given the state h after token t-1, token t updates it in place,
//
//   Delta   = softplus(delta + bias)
//   h[n]    = exp(Delta A[n]) h[n] + Delta B[n] u
//   y       = (sum_n C[n] h[n] + D u) * silu(z)
//
// This pass reads and writes the whole state once per token, so it is bound
// by HBM bandwidth on the state; each thread owns four consecutive states
// (one 16-byte access) and reads their A, B and C as one vector each when
// aligned, and the lanes of a row reduce y with cross-lane shuffles (state
// sizes that are not a multiple of 4: one thread per row).
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

template <typename T> __device__ __forceinline__ float ld1(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld1<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}
template <typename T> __device__ __forceinline__ void st1(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void st1<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st1<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

// Four consecutive elements (16-byte aligned for fp32, 8-byte for bf16).
template <typename T> __device__ __forceinline__ void ld4(const T* p, float v[4]);
template <> __device__ __forceinline__ void ld4<float>(const float* p, float v[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
template <> __device__ __forceinline__ void ld4<uint16_t>(const uint16_t* p, float v[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = bf16lo(q.x); v[1] = bf16hi(q.x); v[2] = bf16lo(q.y); v[3] = bf16hi(q.y);
}

template <bool SP>
__device__ __forceinline__ float delta_log2(float dl, float bias) {
    const float vl = __builtin_fmaf(dl, kLog2e, bias * kLog2e);
    return SP ? softplus_log2(vl) : vl;
}

__device__ __forceinline__ float silu(float z) { return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }

// Sum over the Q lanes of an aligned group (Q a power of two, at most 64).
template <int Q>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = 1; o < Q; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Mamba-1: row = (batch, channel), N states, Q = N/4 threads per row.
template <typename Tin, typename Tout, bool SP, int Q>
__global__ __launch_bounds__(256) void m1_step_kernel(StepArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t rows = a.batch * a.dim;
    const int64_t row_raw = gid / Q;
    const bool ok = row_raw < rows;
    const int64_t row = ok ? row_raw : rows - 1;
    const int qi = (int)(gid % Q);
    const int64_t b = row / a.dim;
    const int64_t d = row - b * a.dim;
    const int N = a.N;
    const Tin* U = reinterpret_cast<const Tin*>(a.u);
    const Tin* DL = reinterpret_cast<const Tin*>(a.delta);
    const Tin* Bm = reinterpret_cast<const Tin*>(a.B);
    const Tin* Cm = reinterpret_cast<const Tin*>(a.C);
    const float uu = ld1(U, row);
    const float w = SP ? delta_log2<true>(ld1(DL, row), a.bias ? a.bias[d] : 0.0f)
                       : delta_log2<false>(ld1(DL, row), a.bias ? a.bias[d] : 0.0f);
    const float x = (w * kLn2) * uu;   // Delta u
    float acc = 0.0f;
    float4* st = reinterpret_cast<float4*>(a.state + row * N) + qi;
    float4 h = *st;
    float* hv = reinterpret_cast<float*>(&h);
    float Av[4], Bv[4], Cv[4];
    if (a.vec) {
        ld4(a.A + d * N + 4 * qi, Av);
        ld4(Bm + b * N + 4 * qi, Bv);
        ld4(Cm + b * N + 4 * qi, Cv);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Av[i] = a.A[d * N + 4 * qi + i];
            Bv[i] = ld1(Bm, b * N + 4 * qi + i);
            Cv[i] = ld1(Cm, b * N + 4 * qi + i);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        hv[i] = __builtin_fmaf(fast_exp2(w * Av[i]), hv[i], x * Bv[i]);
        acc = __builtin_fmaf(Cv[i], hv[i], acc);
    }
    if (ok) *st = h;
    acc = group_sum<Q>(acc);
    if (!ok) return;
    if (qi == 0) {
        float yv = a.D ? __builtin_fmaf(a.D[d], uu, acc) : acc;
        if (a.z) yv *= silu(ld1(reinterpret_cast<const Tin*>(a.z), row));
        st1(reinterpret_cast<Tout*>(a.y), row, yv);
    }
}

// Mamba-1 with N not a multiple of 4: one thread per row.
template <typename Tin, typename Tout, bool SP>
__global__ __launch_bounds__(256) void m1_step_rows_kernel(StepArgs a) {
    const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= a.batch * a.dim) return;
    const int64_t b = row / a.dim;
    const int64_t d = row - b * a.dim;
    const int N = a.N;
    const Tin* Bm = reinterpret_cast<const Tin*>(a.B) + b * N;
    const Tin* Cm = reinterpret_cast<const Tin*>(a.C) + b * N;
    const float uu = ld1(reinterpret_cast<const Tin*>(a.u), row);
    const float dl = ld1(reinterpret_cast<const Tin*>(a.delta), row);
    const float w = delta_log2<SP>(dl, a.bias ? a.bias[d] : 0.0f);
    const float x = (w * kLn2) * uu;
    float acc = 0.0f;
    float* st = a.state + row * N;
    for (int n = 0; n < N; ++n) {
        const float hn = __builtin_fmaf(fast_exp2(w * a.A[d * N + n]), st[n], x * ld1(Bm, n));
        st[n] = hn;
        acc = __builtin_fmaf(ld1(Cm, n), hn, acc);
    }
    float yv = a.D ? __builtin_fmaf(a.D[d], uu, acc) : acc;
    if (a.z) yv *= silu(ld1(reinterpret_cast<const Tin*>(a.z), row));
    st1(reinterpret_cast<Tout*>(a.y), row, yv);
}

// Mamba-2: row = (batch, head, channel), scalar A per head, B/C per group.
template <typename Tin, typename Tout, bool SP, int Q, int E>
__global__ __launch_bounds__(256) void m2_step_kernel(StepArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t rows = a.batch * a.H * a.P;
    const int64_t row_raw = gid / Q;
    const bool ok = row_raw < rows;
    const int64_t row = ok ? row_raw : rows - 1;
    const int qi = (int)(gid % Q);
    const int64_t bh = row / a.P;
    const int64_t b = bh / a.H;
    const int64_t h = bh - b * a.H;
    const int64_t grp = h / (a.H / a.G);
    const int N = a.N;
    const Tin* X = reinterpret_cast<const Tin*>(a.u);
    const Tin* DT = reinterpret_cast<const Tin*>(a.delta);
    const Tin* Bm = reinterpret_cast<const Tin*>(a.B) + (b * a.G + grp) * N;
    const Tin* Cm = reinterpret_cast<const Tin*>(a.C) + (b * a.G + grp) * N;
    float4* st = reinterpret_cast<float4*>(a.state + row * N) + qi * (E / 4);
    float4 s[E / 4];
#pragma unroll
    for (int k = 0; k < E / 4; ++k) s[k] = st[k];
    const float xx = ld1(X, row);
    const float w = SP ? delta_log2<true>(ld1(DT, bh), a.bias ? a.bias[h] : 0.0f)
                       : delta_log2<false>(ld1(DT, bh), a.bias ? a.bias[h] : 0.0f);
    const float dA = fast_exp2(w * a.A[h]);
    const float x = (w * kLn2) * xx;
    float acc = 0.0f;
    float* sv = reinterpret_cast<float*>(&s[0]);
    float Bv[E], Cv[E];
    if (a.vec) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) {
            ld4(Bm + E * qi + 4 * k, Bv + 4 * k);
            ld4(Cm + E * qi + 4 * k, Cv + 4 * k);
        }
    } else {
#pragma unroll
        for (int i = 0; i < E; ++i) {
            Bv[i] = ld1(Bm, E * qi + i);
            Cv[i] = ld1(Cm, E * qi + i);
        }
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {
        sv[i] = __builtin_fmaf(dA, sv[i], x * Bv[i]);
        acc = __builtin_fmaf(Cv[i], sv[i], acc);
    }
    if (ok) {
#pragma unroll
        for (int k = 0; k < E / 4; ++k) st[k] = s[k];
    }
    acc = group_sum<Q>(acc);
    if (!ok) return;
    if (qi == 0) {
        float yv = a.D ? __builtin_fmaf(a.D[h], xx, acc) : acc;
        if (a.z) yv *= silu(ld1(reinterpret_cast<const Tin*>(a.z), row));
        st1(reinterpret_cast<Tout*>(a.y), row, yv);
    }
}

template <typename Tin, typename Tout, bool SP, int Q>
hipError_t launch_q(const StepArgs& a, int64_t rows, hipStream_t stream, bool mamba2) {
    const int64_t threads = rows * Q;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (mamba2) {
        KTime kt("m2_step", stream);
        hipLaunchKernelGGL((m2_step_kernel<Tin, Tout, SP, Q, 4>), dim3(blocks), dim3(256), 0, stream, a);
    } else {
        KTime kt("m1_step", stream);
        hipLaunchKernelGGL((m1_step_kernel<Tin, Tout, SP, Q>), dim3(blocks), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

template <typename Tin, typename Tout, bool SP, int Q>
hipError_t launch_q8(const StepArgs& a, int64_t rows, hipStream_t stream) {
    const int64_t threads = rows * Q;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    KTime kt("m2_step", stream);
    hipLaunchKernelGGL((m2_step_kernel<Tin, Tout, SP, Q, 8>), dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename Tin, typename Tout, bool SP>
hipError_t launch_sp(const StepArgs& a, hipStream_t stream, bool mamba2) {
    const int64_t rows = mamba2 ? a.batch * a.H * a.P : a.batch * a.dim;
    switch (a.N) {
        case 4: return launch_q<Tin, Tout, SP, 1>(a, rows, stream, mamba2);
        case 8: return launch_q<Tin, Tout, SP, 2>(a, rows, stream, mamba2);
        case 16: return launch_q<Tin, Tout, SP, 4>(a, rows, stream, mamba2);
        case 32: return launch_q<Tin, Tout, SP, 8>(a, rows, stream, mamba2);
        case 64: if (mamba2) return launch_q8<Tin, Tout, SP, 8>(a, rows, stream);
                 return launch_q<Tin, Tout, SP, 16>(a, rows, stream, mamba2);
        case 128: if (mamba2) return launch_q8<Tin, Tout, SP, 16>(a, rows, stream);
                  return launch_q<Tin, Tout, SP, 32>(a, rows, stream, mamba2);
        default:
            if (mamba2 || a.N < 1 || a.N > 16) return hipErrorInvalidValue;
            {
                KTime kt("m1_step", stream);
                hipLaunchKernelGGL((m1_step_rows_kernel<Tin, Tout, SP>), dim3((unsigned)((rows + 255) / 256)),
                                   dim3(256), 0, stream, a);
            }
            return hipGetLastError();
    }
}

template <typename Tin, typename Tout>
hipError_t launch_dt(const StepArgs& a, hipStream_t stream, bool mamba2) {
    return a.softplus ? launch_sp<Tin, Tout, true>(a, stream, mamba2) : launch_sp<Tin, Tout, false>(a, stream, mamba2);
}

}  // namespace

hipError_t launch_step(const StepArgs& a, int in_bf16, int out_bf16, int mamba2, hipStream_t stream) {
    if (in_bf16 && out_bf16) return launch_dt<uint16_t, uint16_t>(a, stream, mamba2 != 0);
    if (in_bf16) return launch_dt<uint16_t, float>(a, stream, mamba2 != 0);
    if (out_bf16) return launch_dt<float, uint16_t>(a, stream, mamba2 != 0);
    return launch_dt<float, float>(a, stream, mamba2 != 0);
}

}  // namespace selscan
