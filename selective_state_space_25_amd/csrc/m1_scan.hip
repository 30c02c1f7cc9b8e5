// m1_scan.hip -- Mamba-1 selective scan kernels for gfx950.
//
// The method (the update of section 2.2 of the "Understanding Mamba and
// Selective State Space Models (SSMs)" blog, the read-out of its section 2.1,
// the selective SSM layer of the Mamba README):
//
//   Delta_t = softplus(delta_t + bias_d)
//   h_t[n]  = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t B_t[n] u_t,   h_{-1} = 0
//   y_t     = (sum_n C_t[n] h_t[n] + D_d u_t) * silu(z_t)
//
// Work layout.  A workgroup is one wave; lane l owns channel ("row") d0 + l of
// one batch and keeps its 16 fp32 states in registers, walking its tokens in
// order.  All lanes of the wave read the same B_t and C_t, so they come from
// an fp32 copy laid out [batch][token][B0..B15, C0..C15] through scalar loads
// (the next token's are requested while the current one is computed) and
// enter the FMAs as SGPR operands: the sweep needs no LDS and no barrier.
// u, delta and z arrive as 32-token runs per lane (64 contiguous bytes per
// row for bf16, whole memory sectors), the next run requested before the
// current one is processed and converted only when used.  y is written as
// contiguous 16-byte pieces per lane.
//
// Long sequences are cut into G chunks so that enough waves exist to fill
// the 256 CUs: a summary pass computes, per chunk, the end state from a zero
// start and the chunk's sum of Delta; a carry pass folds the summaries in
// order (h_in(g+1) = exp(A sum Delta_g) h_in(g) + b_g); the output pass then
// rescans each chunk from its true carry-in.  G = 1 is a single pass.
//
// Two decay paths, chosen per wave at run time:
//  - general A: exp(Delta A[n]) = 2^(w A[n]) per update, w = Delta / ln2;
//  - structured A (A[d,n] == fl32((n+1) A[d,0]) for every n, as for the
//    S4D-real initialisation -(n+1), also when scaled per channel): then
//    exp(Delta A[n]) = r^(n+1), r = 2^(w A[d,0]): one exp per token, one
//    multiply per update.  This path also keeps the state divided by
//    sigma_t = Delta_t u_t / ln2 (k = h / (ln2 sigma)), which makes the input
//    term Delta B u equal to B itself:
//        k_t[n] = (sigma_{t-1} / sigma_t) r^(n+1) k_{t-1}[n] + B_t[n]
//        y_t    = (sigma_t sum_n C_t[n] k_t[n] + D u_t / ln2) * ln2 * silu(z_t)
//    A token where some lane's sigma_t is zero, tiny, huge or not finite
//    takes the general form of the update for that token (sigma kept from the
//    previous token and B scaled by sigma_t / sigma_kept), so zeros, NaN and
//    Inf behave as in the plain recurrence.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

constexpr int kRows = 64;       // channels per workgroup = lanes of the wave
constexpr int kNS = 16;         // states per channel (padded)
constexpr int kT = 32;          // tokens per tile
constexpr float kSigLo = 8.673617379884035e-19f;   // 2^-60
constexpr float kSigHi = 1.152921504606847e18f;    // 2^60

typedef __attribute__((address_space(4))) const float* cfptr;

// lgkmcnt(0), vmcnt and expcnt left at their maxima
__device__ __forceinline__ void wait_scalar_loads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ bool wave_all(bool p) { return __builtin_amdgcn_ballot_w64(!p) == 0; }

// A pointer whose value is the same in every lane, held in SGPRs.
__device__ __forceinline__ const float* uniform_ptr(const float* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo);
}

template <typename T> struct Tok;
template <> struct Tok<float> {
    static constexpr int kWords = kT;        // 32-bit words per 32-token run
    static __device__ __forceinline__ float get(const uint32_t* w, int j) { return __uint_as_float(w[j]); }
    static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
};
template <> struct Tok<uint16_t> {
    static constexpr int kWords = kT / 2;
    static __device__ __forceinline__ float get(const uint32_t* w, int j) {
        return (j & 1) ? bf16hi(w[j >> 1]) : bf16lo(w[j >> 1]);
    }
    static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
};

// One 32-token run of one row as raw words.
template <typename T>
struct Run {
    uint32_t w[Tok<T>::kWords];
    __device__ __forceinline__ void load_vec(const T* p) {
        const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int i = 0; i < Tok<T>::kWords / 4; ++i) {
            const uint4 x = q[i];
            w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z; w[4 * i + 3] = x.w;
        }
    }
    __device__ __forceinline__ float operator[](int j) const { return Tok<T>::get(w, j); }
};

template <typename T> struct Out;
template <> struct Out<float> {
    static __device__ __forceinline__ void st4(float* p, const float* v) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
    static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Out<uint16_t> {
    static __device__ __forceinline__ void st4(uint16_t* p, const float* v) {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
    static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// The per-row constants and state of one lane.
struct Lane {
    float k[kNS];
    float Ar[kNS];
    float A0, bias_l, Dv, Dp;
    float sig_prev;   // structured path: h = ln2 * sig_prev * k
    float wsum;       // summary pass: sum of w over the chunk
};

// One token of the sweep.  bc holds the token's B (bc[0..16)) and C
// (bc[16..32)).  Returns the read-out before the gate (output pass).
template <int MODE, bool STRUCT>
__device__ __forceinline__ float token(Lane& L, const float* bc, float uu, float dl, int softplus) {
    const float vl = __builtin_fmaf(dl, kLog2e, L.bias_l);
    const float w = softplus ? softplus_log2(vl) : vl;
    if (MODE == 1) L.wsum += w;
    float acc0 = 0.0f, acc1 = 0.0f;
    if constexpr (STRUCT) {
        const float sig = w * uu;
        const float r = fast_exp2(w * L.A0);
        const bool ok = fabsf(sig) >= kSigLo && fabsf(sig) <= kSigHi;
        if (wave_all(ok)) {
            float q = L.sig_prev * fast_rcp(sig) * r;
#pragma unroll
            for (int n = 0; n < kNS; n += 2) {
                L.k[n] = __builtin_fmaf(q, L.k[n], bc[n]);
                q *= r;
                L.k[n + 1] = __builtin_fmaf(q, L.k[n + 1], bc[n + 1]);
                q *= r;
                if (MODE == 0) {
                    acc0 = __builtin_fmaf(bc[kNS + n], L.k[n], acc0);
                    acc1 = __builtin_fmaf(bc[kNS + n + 1], L.k[n + 1], acc1);
                }
            }
            L.sig_prev = sig;
        } else {
            const float sig_new = ok ? sig : L.sig_prev;
            const float c = sig / sig_new;
            float q = (L.sig_prev / sig_new) * r;
#pragma unroll
            for (int n = 0; n < kNS; ++n) {
                L.k[n] = __builtin_fmaf(q, L.k[n], c * bc[n]);
                q *= r;
                if (MODE == 0) acc0 = __builtin_fmaf(bc[kNS + n], L.k[n], acc0);
            }
            L.sig_prev = sig_new;
        }
        if (MODE == 0) return __builtin_fmaf(L.sig_prev, acc0 + acc1, L.Dp * uu);
        return 0.0f;
    } else {
        const float x = (w * kLn2) * uu;   // Delta u
#pragma unroll
        for (int n = 0; n < kNS; n += 2) {
            const float dA0 = fast_exp2(w * L.Ar[n]);
            const float dA1 = fast_exp2(w * L.Ar[n + 1]);
            L.k[n] = __builtin_fmaf(dA0, L.k[n], x * bc[n]);
            L.k[n + 1] = __builtin_fmaf(dA1, L.k[n + 1], x * bc[n + 1]);
            if (MODE == 0) {
                acc0 = __builtin_fmaf(bc[kNS + n], L.k[n], acc0);
                acc1 = __builtin_fmaf(bc[kNS + n + 1], L.k[n + 1], acc1);
            }
        }
        if (MODE == 0) return __builtin_fmaf(L.Dv, uu, acc0 + acc1);
        return 0.0f;
    }
}

// The chunk [t_begin, t_end) of one wave's 64 rows.  MODE 0: output pass.
// MODE 1: summary pass.
template <typename Tin, typename Tout, int MODE, bool STRUCT>
__device__ __forceinline__ void run_chunk(const M1Args& a, int64_t b, int64_t d0, int g) {
    const int lane = threadIdx.x;
    const bool row_ok = d0 + lane < a.dim;
    const int64_t d = row_ok ? d0 + lane : a.dim - 1;
    const int64_t row = b * a.dim + d;
    const int64_t t_begin = (int64_t)g * a.chunk;
    const int64_t t_end = min<int64_t>(a.L, t_begin + a.chunk);
    const bool has_z = MODE == 0 && a.z != nullptr;
    const bool vec = a.vec_ok != 0;

    const Tin* urow = reinterpret_cast<const Tin*>(a.u) + row * a.L;
    const Tin* drow = reinterpret_cast<const Tin*>(a.delta) + row * a.L;
    const Tin* zrow = has_z ? reinterpret_cast<const Tin*>(a.z) + row * a.L : urow;
    Tout* yrow = reinterpret_cast<Tout*>(a.y) + row * a.L;

    Lane L;
    L.bias_l = (a.bias ? a.bias[d] : 0.0f) * kLog2e;
#pragma unroll
    for (int n = 0; n < kNS; ++n) L.Ar[n] = (n < a.N) ? a.A[d * a.N + n] : 0.0f;
    L.A0 = L.Ar[0];
    L.Dv = (MODE == 0 && a.D) ? a.D[d] : 0.0f;
    L.Dp = L.Dv * kInvLn2;
    if (MODE == 0 && g > 0) {
        const float* cin = a.ws_state + (row * a.G + g) * kNS;
#pragma unroll
        for (int n = 0; n < kNS; ++n) L.k[n] = cin[n];
    } else {
#pragma unroll
        for (int n = 0; n < kNS; ++n) L.k[n] = 0.0f;
    }
    L.sig_prev = kInvLn2;
    L.wsum = 0.0f;
    // gate factor: the structured path carries an extra ln2
    const float gscale = STRUCT ? kInvLn2 : 1.0f;
    const float nogate = STRUCT ? kLn2 : 1.0f;

    // this batch's B/C, 32 floats per token; the address is wave-uniform
    const float* bcb = a.bcq + (b * a.L) * (2 * kNS);

    // Full 32-token tiles: raw words of the next tile are requested first.
    const int64_t t_full_end = vec ? t_begin + ((t_end - t_begin) / kT) * kT : t_begin;
    Run<Tin> ru, rd, rz;
    if (t_begin < t_full_end) {
        ru.load_vec(urow + t_begin);
        rd.load_vec(drow + t_begin);
        if (MODE == 0) rz.load_vec(zrow + t_begin);
    }
    for (int64_t t0 = t_begin; t0 < t_full_end; t0 += kT) {
        const int64_t tn = (t0 + kT < t_full_end) ? t0 + kT : t0;   // clamped, always in bounds
        Run<Tin> nu, nd, nz;
        nu.load_vec(urow + tn);
        nd.load_vec(drow + tn);
        if (MODE == 0) nz.load_vec(zrow + tn);
        // B/C of token j + 1 are requested while token j is computed
        const cfptr bct = (cfptr)uniform_ptr(bcb + t0 * (2 * kNS));
        float bcur[2 * kNS];
#pragma unroll
        for (int e = 0; e < 2 * kNS; ++e) bcur[e] = bct[e];
        float yv[4];
#pragma unroll
        for (int j = 0; j < kT; ++j) {
            // keep each token's scalar loads where they are: hoisting them
            // across tokens would exhaust the SGPRs and spill
            __builtin_amdgcn_sched_barrier(0);
            wait_scalar_loads();
            float bnxt[2 * kNS];
            if (j + 1 < kT) {
#pragma unroll
                for (int e = 0; e < 2 * kNS; ++e) bnxt[e] = bct[(j + 1) * (2 * kNS) + e];
            }
            const float pre = token<MODE, STRUCT>(L, bcur, ru[j], rd[j], a.softplus);
            if (MODE == 0) {
                yv[j & 3] = pre * (has_z ? silu_scaled(rz[j], gscale) : nogate);
                if ((j & 3) == 3 && row_ok) Out<Tout>::st4(yrow + t0 + j - 3, yv);
            }
            if (j + 1 < kT) {
#pragma unroll
                for (int e = 0; e < 2 * kNS; ++e) bcur[e] = bnxt[e];
            }
        }
        ru = nu;
        rd = nd;
        if (MODE == 0) rz = nz;
    }
    // Remaining tokens (a ragged tail, or every token when rows are not
    // 16-byte aligned), one at a time.
    for (int64_t t = t_full_end; t < t_end; ++t) {
        const cfptr bc = (cfptr)(bcb + t * (2 * kNS));
        float bcur[2 * kNS];
#pragma unroll
        for (int e = 0; e < 2 * kNS; ++e) bcur[e] = bc[e];
        const float uu = Tok<Tin>::ld(urow, t);
        const float dl = Tok<Tin>::ld(drow, t);
        const float pre = token<MODE, STRUCT>(L, bcur, uu, dl, a.softplus);
        if (MODE == 0 && row_ok) {
            const float yy = pre * (has_z ? silu_scaled(Tok<Tin>::ld(zrow, t), gscale) : nogate);
            Out<Tout>::st(yrow, t, yy);
        }
    }

    if (!row_ok) return;
    const float hs = STRUCT ? kLn2 * L.sig_prev : 1.0f;
    if (MODE == 1) {
        float* dst = a.ws_state + (row * a.G + g) * kNS;
#pragma unroll
        for (int n = 0; n < kNS; ++n) dst[n] = hs * L.k[n];
        a.ws_w[row * a.G + g] = L.wsum;
    } else if (g == a.G - 1 && a.last) {
#pragma unroll
        for (int n = 0; n < kNS; ++n)
            if (n < a.N) a.last[row * a.N + n] = hs * L.k[n];
    }
}

// True when every state of channel d satisfies A[d,n] == fl32((n+1) A[d,0]).
__device__ __forceinline__ bool row_is_structured(const M1Args& a, int64_t d) {
    const float A0 = a.A[d * a.N];
    bool s = true;
    for (int n = 1; n < a.N; ++n) s = s && (a.A[d * a.N + n] == (float)(n + 1) * A0);
    return s;
}

template <typename Tin, typename Tout, int MODE>
__global__ __launch_bounds__(kRows) void m1_scan_kernel(M1Args a) {
    const int64_t blocks_per_batch = (a.dim + kRows - 1) / kRows;
    const int64_t b = blockIdx.x / blocks_per_batch;
    const int64_t d0 = (blockIdx.x - b * blocks_per_batch) * kRows;
    const int g = blockIdx.y;
    const int64_t d = min<int64_t>(d0 + threadIdx.x, a.dim - 1);
    // the structured path needs every one of the 16 register states to be real
    const bool structured = !a.force_general && a.N == kNS && wave_all(row_is_structured(a, d));
    if (structured)
        run_chunk<Tin, Tout, MODE, true>(a, b, d0, g);
    else
        run_chunk<Tin, Tout, MODE, false>(a, b, d0, g);
}

// B, C [batch, N, L] -> fp32 [batch, L, (B0..B15, C0..C15)] (zeros past N)
template <typename Tin>
__global__ __launch_bounds__(256) void m1_bc_kernel(M1Args a) {
    const int64_t total = a.batch * a.L;
    const Tin* B = reinterpret_cast<const Tin*>(a.B);
    const Tin* C = reinterpret_cast<const Tin*>(a.C);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = i / a.L;
        const int64_t t = i - b * a.L;
        float v[2 * kNS];
#pragma unroll
        for (int n = 0; n < kNS; ++n) {
            v[n] = n < a.N ? Tok<Tin>::ld(B, (b * a.N + n) * a.L + t) : 0.0f;
            v[kNS + n] = n < a.N ? Tok<Tin>::ld(C, (b * a.N + n) * a.L + t) : 0.0f;
        }
        float4* o = reinterpret_cast<float4*>(a.bcq + i * (2 * kNS));
#pragma unroll
        for (int q = 0; q < 2 * kNS / 4; ++q) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
}

// Carry pass: one thread per (row, n).  Turns the per-chunk end states b_g
// (slot g) into carries-in h_in(g) (slot g), in chunk order:
//   h_in(0) = 0,   h_in(g+1) = 2^(A[d,n] W_g) h_in(g) + b_g.
__global__ __launch_bounds__(256) void m1_carry_kernel(M1Args a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t rows = a.batch * a.dim;
    if (idx >= rows * kNS) return;
    const int64_t row = idx / kNS;
    const int n = (int)(idx - row * kNS);
    const int64_t d = row % a.dim;
    const float An = (n < a.N) ? a.A[d * a.N + n] : 0.0f;
    float h = 0.0f;
    float* st = a.ws_state + row * a.G * kNS + n;
    const float* W = a.ws_w + row * a.G;
    for (int g = 0; g < a.G; ++g) {
        const float bg = (g < a.G - 1) ? st[(int64_t)g * kNS] : 0.0f;
        st[(int64_t)g * kNS] = h;
        if (g < a.G - 1) h = __builtin_fmaf(fast_exp2(An * W[g]), h, bg);
    }
}

template <typename Tin, typename Tout>
hipError_t launch_dt(const M1Args& a, hipStream_t stream) {
    const int64_t bc_blocks = std::min<int64_t>((a.batch * a.L + 255) / 256, 16384);
    {
        KTime kt("m1_bc_convert", stream);
        hipLaunchKernelGGL((m1_bc_kernel<Tin>), dim3((unsigned)bc_blocks), dim3(256), 0, stream, a);
    }
    const int64_t blocks_per_batch = (a.dim + kRows - 1) / kRows;
    const unsigned gx = (unsigned)(blocks_per_batch * a.batch);
    if (a.G > 1) {
        {
            KTime kt("m1_scan_summary", stream);
            hipLaunchKernelGGL((m1_scan_kernel<Tin, Tout, 1>), dim3(gx, (unsigned)(a.G - 1)), dim3(kRows), 0,
                               stream, a);
        }
        const int64_t threads = a.batch * a.dim * kNS;
        KTime kt("m1_chunk_carry", stream);
        hipLaunchKernelGGL(m1_carry_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
    }
    KTime kt("m1_scan_output", stream);
    hipLaunchKernelGGL((m1_scan_kernel<Tin, Tout, 0>), dim3(gx, (unsigned)a.G), dim3(kRows), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int m1_padded_states(int) { return kNS; }
int m1_rows_per_block() { return kRows; }
int m1_waves_per_block() { return 1; }
size_t m1_bc_bytes(int64_t batch, int64_t L) { return (size_t)batch * L * 2 * kNS * sizeof(float); }

hipError_t launch_m1(const M1Args& a, int in_bf16, int out_bf16, hipStream_t stream) {
    if (in_bf16 && out_bf16) return launch_dt<uint16_t, uint16_t>(a, stream);
    if (in_bf16) return launch_dt<uint16_t, float>(a, stream);
    if (out_bf16) return launch_dt<float, uint16_t>(a, stream);
    return launch_dt<float, float>(a, stream);
}

}  // namespace selscan
