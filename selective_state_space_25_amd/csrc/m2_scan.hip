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
// Work layout.  A workgroup owns 64 channels p of one (batch, head) and one
// time chunk, with N/16 waves; wave w keeps states 16w..16w+15 of every
// channel (lane = channel) in registers.  Each 16-token tile runs in three
// phases separated by barriers:
//   A  per-(channel, token) scalars, lanes along p so that x and z loads are
//      contiguous: Delta, sigma (below), the gate, the skip term.
//   B  the sweep: B_t and C_t are the same for every lane of the wave, read
//      as scalar loads from an fp32 copy [batch, L, G, (B[0..N), C[0..N))]
//      and used as SGPR operands; each wave writes its partial read-out.
//   C  partial sums added, skip and gate applied, y stored along p.
//
// The decay exp(Delta A[h]) is the same for all n, and the state is kept
// divided by sigma_t = Delta_t x_t / ln2 (k = s / (ln2 sigma)):
//   k_t[n] = (sigma_{t-1}/sigma_t) 2^(w_t A[h]) k_{t-1}[n] + B_t[n]
// so each state costs one FMA for the update and one for the read-out.
// Where sigma_t is zero, tiny, huge or not finite it is replaced by 1 and B
// is scaled by the true sigma_t for that token (the plain recurrence); a tile
// holding such a token runs the scaled form throughout.
//
// As for Mamba-1, long sequences are split into chunks: summary pass, carry
// pass, output pass from the true carry-in.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

constexpr int kP = 64;        // channels per workgroup (lane = channel)
constexpr int kSPW = 16;      // states per wave
constexpr int kT = 16;        // tokens per tile
constexpr int kAccStride = kP + 1;
constexpr float kSigLo = 8.673617379884035e-19f;  // 2^-60
constexpr float kSigHi = 1.152921504606847e18f;   // 2^60

typedef __attribute__((address_space(4))) const float* cfptr;

template <typename T> __device__ __forceinline__ float ldv(const T* p, int64_t i);
template <> __device__ __forceinline__ float ldv<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldv<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
template <typename T> __device__ __forceinline__ void stv(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void stv<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void stv<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

template <int NW>
struct Smem2 {
    float sig[kT][kP];                 // sigma per (token, channel)
    float c[kT][kP];                   // B scale where sigma was replaced
    float dA[kT];                      // 2^(w A[h]) per token
    float acc[NW][kT][kAccStride];     // partial read-outs
    float sig_last[kP];
    float wpart[NW];
};

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
__global__ __launch_bounds__(kP * (N / kSPW)) void m2_scan_kernel(M2Args a) {
    constexpr int NW = N / kSPW;
    constexpr int kPer = kT / NW;      // tokens per thread in phases A and C
    __shared__ Smem2<NW> sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;

    const int64_t pblocks = (a.P + kP - 1) / kP;
    const int64_t bh = blockIdx.x / pblocks;     // batch * H + head
    const int64_t pb = blockIdx.x - bh * pblocks;
    const int64_t b = bh / a.H;
    const int64_t h = bh - b * a.H;
    const int64_t p_raw = pb * kP + lane;
    const bool p_ok = p_raw < a.P;
    const int64_t p = p_ok ? p_raw : a.P - 1;
    const int g = blockIdx.y;
    const int64_t grp = h / (a.H / a.G);
    const int64_t t_begin = (int64_t)g * a.chunk;
    const int64_t t_end = min<int64_t>(a.L, t_begin + a.chunk);
    // phase A/C: channel = lane, tokens [wave * kPer, wave * kPer + kPer) of the tile
    const int aj0 = wave * kPer;

    const Tin* X = reinterpret_cast<const Tin*>(a.x);
    const Tin* DT = reinterpret_cast<const Tin*>(a.dt);
    const Tin* Z = reinterpret_cast<const Tin*>(a.z);
    Tout* Y = reinterpret_cast<Tout*>(a.y);
    const bool has_z = MODE == 0 && a.z != nullptr;
    const float Ah = a.A[h];
    const float bias_l = (a.dt_bias ? a.dt_bias[h] : 0.0f) * kLog2e;
    const float Dp = (MODE == 0 && a.D) ? a.D[h] * kInvLn2 : 0.0f;
    const int64_t unit = (b * a.H + h) * a.P + p;   // (batch, head, channel)

    float k[kSPW];
    if (MODE == 0 && g > 0) {
        const float* cin = a.ws_state + (unit * a.chunks + g) * N + wave * kSPW;
#pragma unroll
        for (int i = 0; i < kSPW; ++i) k[i] = cin[i];
    } else if (MODE == 0 && a.h0) {
        // chunk 0 starts from the caller's state (k = h while sig_prev = 1/ln2)
        const float* cin = a.h0 + unit * N + wave * kSPW;
#pragma unroll
        for (int i = 0; i < kSPW; ++i) k[i] = cin[i];
    } else {
#pragma unroll
        for (int i = 0; i < kSPW; ++i) k[i] = 0.0f;
    }
    float sig_prev = kInvLn2;   // sweep: sigma of the previous token
    float wsum = 0.0f;

    // this thread's x, dt, z for the current tile; the next tile's are
    // requested before the current one is processed
    float cx[kPer], cdt[kPer], cz[kPer];
    auto fetch = [&](int64_t tt0, float* fx, float* fdt, float* fz) {
        const int nt = (int)min<int64_t>(kT, t_end - tt0);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int jj = aj0 + j;
            const bool live = jj < nt;
            const int64_t bt = b * a.L + tt0 + (live ? jj : 0);
            const int64_t xi = (bt * a.H + h) * a.P + p;
            fx[j] = live ? ldv<Tin>(X, xi) : 0.0f;
            fdt[j] = ldv<Tin>(DT, bt * a.H + h);
            fz[j] = (has_z && live) ? ldv<Tin>(Z, xi) : 0.0f;
        }
    };
    fetch(t_begin, cx, cdt, cz);

    for (int64_t t0 = t_begin; t0 < t_end; t0 += kT) {
        const int ntok = (int)min<int64_t>(kT, t_end - t0);
        float nx[kPer], ndt[kPer], nz[kPer];
        if (t0 + kT < t_end) fetch(t0 + kT, nx, ndt, nz);
        // ------------------------------------------------------------ phase A
        float gate[kPer], dx[kPer], sg[kPer];
        bool slow = false;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int jj = aj0 + j;
            const bool live = jj < ntok;
            const float xv = cx[j];
            const float vl = __builtin_fmaf(cdt[j], kLog2e, bias_l);
            const float w = a.softplus ? softplus_log2(vl) : vl;
            if (MODE == 1 && live) wsum += w;
            const float s = w * xv;
            const bool ok = fabsf(s) >= kSigLo && fabsf(s) <= kSigHi;
            sg[j] = ok ? s : 1.0f;
            slow = slow || (!ok && live);
            sm.sig[jj][lane] = sg[j];
            sm.c[jj][lane] = ok ? 1.0f : s;
            if (lane == 0) sm.dA[jj] = fast_exp2(w * Ah);
            if (MODE == 0) {
                gate[j] = has_z ? silu_scaled(cz[j], kInvLn2) : kLn2;
                dx[j] = Dp * xv;
            }
            if (jj == ntok - 1 && (t0 + jj == t_end - 1)) sm.sig_last[lane] = sg[j];
        }
        const bool tile_slow = __syncthreads_or(slow ? 1 : 0) != 0;
        // ------------------------------------------------------------ phase B
        {
            const cfptr bc0 = (cfptr)(a.ws_bc + ((b * a.L + t0) * a.G + grp) * 2 * N + wave * kSPW);
            const int64_t tstride = a.G * 2 * N;   // floats between consecutive tokens
            if (ntok == kT) {
                float sv[kT], dav[kT], cv[kT];
#pragma unroll
                for (int j = 0; j < kT; ++j) {
                    sv[j] = sm.sig[j][lane];
                    dav[j] = sm.dA[j];
                    cv[j] = tile_slow ? sm.c[j][lane] : 1.0f;
                }
                // B/C of token j+1 are requested while token j is computed;
                // the explicit wait retires exactly the previous request
                float bcur[2 * kSPW];
#pragma unroll
                for (int e = 0; e < kSPW; ++e) {
                    bcur[e] = bc0[e];
                    bcur[kSPW + e] = bc0[N + e];
                }
#pragma unroll
                for (int j = 0; j < kT; ++j) {
                    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                    float bnxt[2 * kSPW];
                    if (j + 1 < kT) {
                        const cfptr bt = bc0 + (int64_t)(j + 1) * tstride;
#pragma unroll
                        for (int e = 0; e < kSPW; ++e) {
                            bnxt[e] = bt[e];
                            bnxt[kSPW + e] = bt[N + e];
                        }
                    }
                    const float q = sig_prev * fast_rcp(sv[j]) * dav[j];
                    sig_prev = sv[j];
                    float acc0 = 0.0f, acc1 = 0.0f;
                    if (!tile_slow) {
#pragma unroll
                        for (int i = 0; i < kSPW; i += 2) {
                            k[i] = __builtin_fmaf(q, k[i], bcur[i]);
                            k[i + 1] = __builtin_fmaf(q, k[i + 1], bcur[i + 1]);
                            acc0 = __builtin_fmaf(bcur[kSPW + i], k[i], acc0);
                            acc1 = __builtin_fmaf(bcur[kSPW + i + 1], k[i + 1], acc1);
                        }
                    } else {
                        const float c = cv[j];
#pragma unroll
                        for (int i = 0; i < kSPW; i += 2) {
                            k[i] = __builtin_fmaf(q, k[i], c * bcur[i]);
                            k[i + 1] = __builtin_fmaf(q, k[i + 1], c * bcur[i + 1]);
                            acc0 = __builtin_fmaf(bcur[kSPW + i], k[i], acc0);
                            acc1 = __builtin_fmaf(bcur[kSPW + i + 1], k[i + 1], acc1);
                        }
                    }
                    if (MODE == 0) sm.acc[wave][j][lane] = acc0 + acc1;
                    if (j + 1 < kT) {
#pragma unroll
                        for (int e = 0; e < 2 * kSPW; ++e) bcur[e] = bnxt[e];
                    }
                }
            } else {
                for (int j = 0; j < ntok; ++j) {
                    const cfptr bt = bc0 + (int64_t)j * tstride;
                    const float sj = sm.sig[j][lane];
                    const float q = sig_prev * fast_rcp(sj) * sm.dA[j];
                    sig_prev = sj;
                    const float c = tile_slow ? sm.c[j][lane] : 1.0f;
                    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
                    for (int i = 0; i < kSPW; i += 2) {
                        k[i] = __builtin_fmaf(q, k[i], c * bt[i]);
                        k[i + 1] = __builtin_fmaf(q, k[i + 1], c * bt[i + 1]);
                        acc0 = __builtin_fmaf(bt[N + i], k[i], acc0);
                        acc1 = __builtin_fmaf(bt[N + i + 1], k[i + 1], acc1);
                    }
                    if (MODE == 0) sm.acc[wave][j][lane] = acc0 + acc1;
                }
            }
        }
        __syncthreads();
        // ------------------------------------------------------------ phase C
        if (MODE == 0) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int jj = aj0 + j;
                if (jj < ntok && p_ok) {
                    float s = 0.0f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) s += sm.acc[w][jj][lane];
                    const float yy = __builtin_fmaf(sg[j], s, dx[j]) * gate[j];
                    stv<Tout>(Y, ((b * a.L + t0 + jj) * a.H + h) * a.P + p, yy);
                }
            }
        }
        // the next tile's phase A rewrites sig/c/dA/acc only after this barrier
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            cx[j] = nx[j];
            cdt[j] = ndt[j];
            cz[j] = nz[j];
        }
    }

    const float hs = kLn2 * sm.sig_last[lane];
    if (MODE == 1) {
        // every lane of a wave saw the same tokens' w: one partial per wave,
        // added in wave order so the sum is the same on every run
        if (lane == 0) sm.wpart[wave] = wsum;
        __syncthreads();
        if (tid == 0) {
            float ws = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) ws += sm.wpart[w];
            a.ws_w[(b * a.H + h) * a.chunks + g] = ws;
        }
        if (p_ok) {
            float* dst = a.ws_state + (unit * a.chunks + g) * N + wave * kSPW;
#pragma unroll
            for (int i = 0; i < kSPW; ++i) dst[i] = hs * k[i];
        }
    } else if (g == a.chunks - 1 && a.last && p_ok) {
        float* dst = a.last + unit * N + wave * kSPW;
#pragma unroll
        for (int i = 0; i < kSPW; ++i) dst[i] = hs * k[i];
    }
}

// Carry pass, one thread per (batch, head, channel, n):
//   h_in(0) = h0 (or 0),  h_in(g+1) = 2^(A[h] W_g) h_in(g) + b_g   (in place).
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
    float hv = a.h0 ? a.h0[unit * a.N + n] : 0.0f;
    for (int g = 0; g < a.chunks; ++g) {
        const float bg = (g < a.chunks - 1) ? st[(int64_t)g * a.N] : 0.0f;
        st[(int64_t)g * a.N] = hv;
        if (g < a.chunks - 1) hv = __builtin_fmaf(fast_exp2(Ah * W[g]), hv, bg);
    }
}

template <typename Tin, typename Tout, int N>
hipError_t launch_n(const M2Args& a, hipStream_t stream) {
    constexpr int threads = kP * (N / kSPW);
    const int64_t total = a.batch * a.L * a.G * a.N;
    const int64_t cblocks = std::min<int64_t>((total + 255) / 256, 65536);
    {
        KTime kt("m2_bc_convert", stream);
        hipLaunchKernelGGL((m2_bc_convert_kernel<Tin>), dim3((unsigned)cblocks), dim3(256), 0, stream, a);
    }
    const int64_t pblocks = (a.P + kP - 1) / kP;
    const unsigned gx = (unsigned)(a.batch * a.H * pblocks);
    if (a.chunks > 1) {
        {
            KTime kt("m2_scan_summary", stream);
            hipLaunchKernelGGL((m2_scan_kernel<Tin, Tout, N, 1>), dim3(gx, (unsigned)(a.chunks - 1)), dim3(threads),
                               0, stream, a);
        }
        const int64_t nthreads = a.batch * a.H * a.P * a.N;
        KTime kt("m2_chunk_carry", stream);
        hipLaunchKernelGGL(m2_carry_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, stream, a);
    }
    KTime kt("m2_scan_output", stream);
    hipLaunchKernelGGL((m2_scan_kernel<Tin, Tout, N, 0>), dim3(gx, (unsigned)a.chunks), dim3(threads), 0, stream, a);
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

int m2_waves_per_block(int64_t N) { return (int)(N / kSPW); }

hipError_t launch_m2(const M2Args& a, int in_bf16, int out_bf16, hipStream_t stream) {
    if (in_bf16 && out_bf16) return launch_dt<uint16_t, uint16_t>(a, stream);
    if (in_bf16) return launch_dt<uint16_t, float>(a, stream);
    if (out_bf16) return launch_dt<float, uint16_t>(a, stream);
    return launch_dt<float, float>(a, stream);
}

}  // namespace selscan
