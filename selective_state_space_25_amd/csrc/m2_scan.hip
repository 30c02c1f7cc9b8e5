// m2_scan.hip -- Mamba-2 multi-head selective scan kernels for gfx950.
//
// Mamba-2 (the Mamba README's Mamba-2 block; the "model-architecture-mamba"
// page's multi-head variant with d_state 128 and headdim 64) keeps the
// selective update of the "Understanding Mamba ..." blog (section 2.2) but
// makes A a scalar per head and shares one Delta per (batch, token, head)
// across the head's P channels, and B/C across the heads of a group:
//
//   Delta_t    = softplus(dt_t[h] + dt_bias[h])
//   s_t[p, n]  = exp(Delta_t A[h]) s_{t-1}[p, n] + Delta_t B_t[g, n] x_t[h, p]
//   y_t[h, p]  = (sum_n C_t[g, n] s_t[p, n] + D[h] x_t[h, p]) * silu(z_t[h, p])
//
// Layout of the work.  One lane owns one channel p of one (batch, head) and
// keeps its N fp32 states in registers; a wave covers 64 channels.  Every
// lane of a wave reads the same B_t and C_t, so they are read as wave-uniform
// scalar loads from an fp32 copy laid out [batch, L, G, 2, N] (made by a
// small conversion kernel) and enter the FMAs as SGPR operands.
//
// Because the decay exp(Delta A[h]) is the same for all n, the state is kept
// divided by sigma_t = Delta_t x_t / ln2 (k = s / (ln2 sigma)):
//   k_t[n] = (sigma_{t-1}/sigma_t) 2^(w_t A[h]) k_{t-1}[n] + B_t[n]
// which leaves one FMA for the update and one for the read-out per state.
// Tokens where some lane's sigma_t is zero, tiny, huge or not finite use the
// general update for that token (sigma kept, B scaled by sigma_t/sigma_kept).
//
// As in the Mamba-1 kernels, long sequences are split into chunks: summary
// pass, carry pass, output pass from the true carry-in.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

constexpr int kWave = 64;
constexpr float kSigLo = 8.673617379884035e-19f;  // 2^-60
constexpr float kSigHi = 1.152921504606847e18f;   // 2^60

template <typename T> __device__ __forceinline__ float ldv(const T* p, int64_t i);
template <> __device__ __forceinline__ float ldv<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldv<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
template <typename T> __device__ __forceinline__ void stv(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void stv<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void stv<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

__device__ __forceinline__ bool wave_all(bool p) { return __builtin_amdgcn_ballot_w64(!p) == 0; }

// B, C [batch, L, G, N] -> fp32 [batch, L, G, 2, N]
template <typename Tin>
__global__ __launch_bounds__(256) void m2_bc_convert_kernel(M2Args a) {
    const int64_t total = a.batch * a.L * a.G * a.N;
    const Tin* B = reinterpret_cast<const Tin*>(a.B);
    const Tin* C = reinterpret_cast<const Tin*>(a.C);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tg = i / a.N;
        const int64_t n = i - tg * a.N;
        a.ws_bc[(tg * 2) * a.N + n] = ldv<Tin>(B, i);
        a.ws_bc[(tg * 2 + 1) * a.N + n] = ldv<Tin>(C, i);
    }
}

// MODE 0: output pass.  MODE 1: summary pass (chunk end state from zero and
// the chunk's sum of w = Delta/ln2).
template <typename Tin, typename Tout, int N, int MODE>
__global__ __launch_bounds__(kWave) void m2_scan_kernel(M2Args a) {
    const int64_t pblocks = (a.P + kWave - 1) / kWave;
    const int64_t bh = blockIdx.x / pblocks;          // batch * H + head
    const int64_t pb = blockIdx.x - bh * pblocks;
    const int64_t b = bh / a.H;
    const int64_t h = bh - b * a.H;
    const int64_t p_raw = pb * kWave + threadIdx.x;
    const bool active = p_raw < a.P;
    const int64_t p = active ? p_raw : a.P - 1;
    const int g = blockIdx.y;
    const int64_t grp = h / (a.H / a.G);
    const int64_t t_begin = (int64_t)g * a.chunk;
    const int64_t t_end = min<int64_t>(a.L, t_begin + a.chunk);

    const Tin* X = reinterpret_cast<const Tin*>(a.x);
    const Tin* DT = reinterpret_cast<const Tin*>(a.dt);
    const Tin* Z = reinterpret_cast<const Tin*>(a.z);
    Tout* Y = reinterpret_cast<Tout*>(a.y);
    const bool has_z = (MODE == 0) && a.z != nullptr;
    const float Ah = a.A[h];
    const float bias_l = (a.dt_bias ? a.dt_bias[h] : 0.0f) * kLog2e;
    const float Dp = (MODE == 0 && a.D) ? a.D[h] * kInvLn2 : 0.0f;
    const int64_t unit = (b * a.H + h) * a.P + p;   // (batch, head, channel)

    float k[N];
    if (MODE == 0 && g > 0) {
        const float* cin = a.ws_state + (unit * a.chunks + g) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) k[n] = cin[n];
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) k[n] = 0.0f;
    }
    float sig_prev = kInvLn2;
    float wsum = 0.0f;

    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t bt = b * a.L + t;
        const float vl = __builtin_fmaf(ldv<Tin>(DT, bt * a.H + h), kLog2e, bias_l);
        const float w = a.softplus ? softplus_log2(vl) : vl;
        if (MODE == 1) wsum += w;
        const int64_t xi = (bt * a.H + h) * a.P + p;
        const float xv = ldv<Tin>(X, xi);
        const float sig = w * xv;
        const float dA = fast_exp2(w * Ah);
        const float* bct = a.ws_bc + ((bt * a.G + grp) * 2) * a.N;  // wave-uniform
        const bool ok = fabsf(sig) >= kSigLo && fabsf(sig) <= kSigHi;
        float acc0 = 0.0f, acc1 = 0.0f;
        if (wave_all(ok)) {
            const float q = sig_prev * fast_rcp(sig) * dA;
#pragma unroll
            for (int n = 0; n < N; n += 2) {
                k[n] = __builtin_fmaf(q, k[n], bct[n]);
                k[n + 1] = __builtin_fmaf(q, k[n + 1], bct[n + 1]);
                if (MODE == 0) {
                    acc0 = __builtin_fmaf(bct[N + n], k[n], acc0);
                    acc1 = __builtin_fmaf(bct[N + n + 1], k[n + 1], acc1);
                }
            }
            sig_prev = sig;
        } else {
            const float sig_new = ok ? sig : sig_prev;
            const float c = sig / sig_new;
            const float q = (sig_prev / sig_new) * dA;
#pragma unroll
            for (int n = 0; n < N; n += 2) {
                k[n] = __builtin_fmaf(q, k[n], c * bct[n]);
                k[n + 1] = __builtin_fmaf(q, k[n + 1], c * bct[n + 1]);
                if (MODE == 0) {
                    acc0 = __builtin_fmaf(bct[N + n], k[n], acc0);
                    acc1 = __builtin_fmaf(bct[N + n + 1], k[n + 1], acc1);
                }
            }
            sig_prev = sig_new;
        }
        if (MODE == 0) {
            float yy = __builtin_fmaf(sig_prev, acc0 + acc1, Dp * xv);
            yy *= has_z ? silu_scaled(ldv<Tin>(Z, xi), kInvLn2) : kLn2;
            if (active) stv<Tout>(Y, xi, yy);
        }
    }

    if (!active) return;
    const float hs = kLn2 * sig_prev;
    if (MODE == 1) {
        float* dst = a.ws_state + (unit * a.chunks + g) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) dst[n] = hs * k[n];
        if (p == 0) a.ws_w[(b * a.H + h) * a.chunks + g] = wsum;
    } else if (g == a.chunks - 1 && a.last) {
        float* dst = a.last + unit * N;
#pragma unroll
        for (int n = 0; n < N; ++n) dst[n] = hs * k[n];
    }
}

// Carry pass, one thread per (batch, head, channel, n):
//   h_in(0) = 0,  h_in(g+1) = 2^(A[h] W_g) h_in(g) + b_g   (in place).
__global__ __launch_bounds__(256) void m2_carry_kernel(M2Args a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = a.batch * a.H * a.P * a.N;
    if (idx >= total) return;
    const int64_t unit = idx / a.N;
    const int64_t n = idx - unit * a.N;
    const int64_t bh = unit / a.P;
    const int64_t h = bh % a.H;
    const float Ah = a.A[h];
    float* st = a.ws_state + unit * a.chunks * a.N + n;
    const float* W = a.ws_w + bh * a.chunks;
    float hv = 0.0f;
    for (int g = 0; g < a.chunks; ++g) {
        const float bg = (g < a.chunks - 1) ? st[(int64_t)g * a.N] : 0.0f;
        st[(int64_t)g * a.N] = hv;
        if (g < a.chunks - 1) hv = __builtin_fmaf(fast_exp2(Ah * W[g]), hv, bg);
    }
}

template <typename Tin, typename Tout, int N>
hipError_t launch_n(const M2Args& a, hipStream_t stream) {
    const int64_t total = a.batch * a.L * a.G * a.N;
    const int64_t cblocks = std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL((m2_bc_convert_kernel<Tin>), dim3((unsigned)cblocks), dim3(256), 0, stream, a);
    const int64_t pblocks = (a.P + kWave - 1) / kWave;
    const unsigned gx = (unsigned)(a.batch * a.H * pblocks);
    if (a.chunks > 1) {
        hipLaunchKernelGGL((m2_scan_kernel<Tin, Tout, N, 1>), dim3(gx, (unsigned)(a.chunks - 1)), dim3(kWave), 0,
                           stream, a);
        const int64_t threads = a.batch * a.H * a.P * a.N;
        hipLaunchKernelGGL(m2_carry_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
    }
    hipLaunchKernelGGL((m2_scan_kernel<Tin, Tout, N, 0>), dim3(gx, (unsigned)a.chunks), dim3(kWave), 0, stream, a);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_dt(const M2Args& a, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_n<Tin, Tout, 16>(a, stream);
        case 32: return launch_n<Tin, Tout, 32>(a, stream);
        case 64: return launch_n<Tin, Tout, 64>(a, stream);
        case 128: return launch_n<Tin, Tout, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_m2(const M2Args& a, int in_bf16, int out_bf16, hipStream_t stream) {
    if (in_bf16 && out_bf16) return launch_dt<uint16_t, uint16_t>(a, stream);
    if (in_bf16) return launch_dt<uint16_t, float>(a, stream);
    if (out_bf16) return launch_dt<float, uint16_t>(a, stream);
    return launch_dt<float, float>(a, stream);
}

}  // namespace selscan
