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
// Layout of the work.  One lane owns one (batch, channel) row and keeps its
// NS fp32 states in registers; it walks its tokens in order.  A workgroup is
// 256 consecutive channels of one batch, so B_t and C_t (shared by every
// channel of a batch) are staged once per 16-token tile in LDS as fp32 and
// read by all lanes with broadcast ds_read_b128.  u, delta and z arrive as
// 16-byte vector loads per lane.
//
// Long sequences are cut into G chunks so that enough waves exist to fill
// the 256 CUs: a summary pass computes, per chunk, the end state from a zero
// start and the chunk's sum of Delta; a carry pass folds the summaries in
// order (h_in(g+1) = exp(A sum Delta_g) h_in(g) + b_g); the output pass then
// rescans each chunk from its true carry-in.  G = 1 is a single pass.
//
// Two decay paths, chosen per workgroup at run time:
//  - general A: exp(Delta A[n]) = 2^(w A[n]) per update, with w = Delta/ln2;
//  - structured A (A[d,n] == fl32((n+1) A[d,0]) for all n, which holds for the
//    S4D-real initialisation -(n+1), also when scaled per channel): then
//    exp(Delta A[n]) = r^(n+1) with r = 2^(w A[d,0]): one exp per token and a
//    multiply per update.  This path also keeps the state divided by
//    sigma_t = Delta_t u_t / ln2 (k_t = h_t / (ln2 sigma_t)), which turns the
//    input term Delta B u into B itself:
//        k_t[n] = (sigma_{t-1}/sigma_t) r^(n+1) k_{t-1}[n] + B_t[n]
//        y_t    = ln2 (sigma_t sum_n C_t[n] k_t[n] + D u_t / ln2)
//    Tokens where some lane's sigma_t is zero, tiny, huge or not finite take
//    the general form of that update (sigma kept from the previous token and
//    B scaled by sigma_t/sigma_kept), so zeros, NaN and Inf behave exactly as
//    in the plain recurrence.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

constexpr int kTile = 16;     // tokens per LDS tile
constexpr int kBlock = 256;   // lanes (channels) per workgroup
constexpr float kSigLo = 8.673617379884035e-19f;   // 2^-60
constexpr float kSigHi = 1.152921504606847e18f;    // 2^60

template <typename T> struct InTraits;
template <> struct InTraits<float> {
    static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
    // 16 consecutive values from a 16-byte aligned address
    static __device__ __forceinline__ void ld16(const float* p, float* v) {
        const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 x = q[i];
            v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
        }
    }
};
template <> struct InTraits<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void ld16(const uint16_t* p, float* v) {
        const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint4 x = q[i];
            v[8 * i + 0] = bf16lo(x.x); v[8 * i + 1] = bf16hi(x.x);
            v[8 * i + 2] = bf16lo(x.y); v[8 * i + 3] = bf16hi(x.y);
            v[8 * i + 4] = bf16lo(x.z); v[8 * i + 5] = bf16hi(x.z);
            v[8 * i + 6] = bf16lo(x.w); v[8 * i + 7] = bf16hi(x.w);
        }
    }
};

template <typename T> struct OutTraits;
template <> struct OutTraits<float> {
    static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
    static __device__ __forceinline__ void st16(float* p, const float* v) {
        float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
};
template <> struct OutTraits<uint16_t> {
    static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
    static __device__ __forceinline__ void st16(uint16_t* p, const float* v) {
        uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            q[i] = make_uint4(pack_bf16x2(v[8 * i], v[8 * i + 1]), pack_bf16x2(v[8 * i + 2], v[8 * i + 3]),
                              pack_bf16x2(v[8 * i + 4], v[8 * i + 5]), pack_bf16x2(v[8 * i + 6], v[8 * i + 7]));
    }
};

// Load tokens [t0, t0 + ntok) of one row into v[0..kTile) (zeros past ntok).
template <typename Tin>
__device__ __forceinline__ void load_row_tile(const Tin* rowp, int64_t t0, int ntok, bool vec, float* v) {
    if (vec && ntok == kTile) {
        InTraits<Tin>::ld16(rowp + t0, v);
    } else {
#pragma unroll
        for (int j = 0; j < kTile; ++j) v[j] = (j < ntok) ? InTraits<Tin>::ld(rowp, t0 + j) : 0.0f;
    }
}

template <typename Tout>
__device__ __forceinline__ void store_row_tile(Tout* rowp, int64_t t0, int ntok, bool vec, const float* v) {
    if (vec && ntok == kTile) {
        OutTraits<Tout>::st16(rowp + t0, v);
    } else {
#pragma unroll
        for (int j = 0; j < kTile; ++j)
            if (j < ntok) OutTraits<Tout>::st(rowp, t0 + j, v[j]);
    }
}

__device__ __forceinline__ bool wave_all(bool p) {
    return __builtin_amdgcn_ballot_w64(!p) == 0;
}

// One chunk of one row.  MODE 0: output pass (writes y, and last_state on
// the final chunk).  MODE 1: summary pass (writes the chunk's end state from
// a zero start and its sum of w = Delta/ln2).
template <typename Tin, typename Tout, int NS, int MODE, bool STRUCT>
__device__ __forceinline__ void scan_chunk(const M1Args& a, float4 (*bc)[2][NS / 4], int b,
                                           int64_t dd, bool active, int64_t t_begin, int64_t t_end,
                                           int g) {
    const int64_t row = (int64_t)b * a.dim + dd;
    const int tid = threadIdx.x;
    const Tin* u_row = reinterpret_cast<const Tin*>(a.u) + row * a.L;
    const Tin* d_row = reinterpret_cast<const Tin*>(a.delta) + row * a.L;
    const Tin* z_row = a.z ? reinterpret_cast<const Tin*>(a.z) + row * a.L : nullptr;
    const Tin* Bg = reinterpret_cast<const Tin*>(a.B) + (int64_t)b * a.N * a.L;
    const Tin* Cg = reinterpret_cast<const Tin*>(a.C) + (int64_t)b * a.N * a.L;
    const bool vec = a.vec_ok != 0;
    const bool has_z = (MODE == 0) && a.z != nullptr;

    const float bias_l = (a.bias ? a.bias[dd] : 0.0f) * kLog2e;
    float Ar[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) Ar[n] = (n < a.N) ? a.A[dd * a.N + n] : 0.0f;
    const float A0 = Ar[0];
    const float Dv = (MODE == 0 && a.D) ? a.D[dd] : 0.0f;
    const float Dp = STRUCT ? Dv * kInvLn2 : Dv;

    float k[NS];
    if (MODE == 0 && g > 0) {
        const float* cin = a.ws_state + (row * a.G + g) * NS;
#pragma unroll
        for (int n = 0; n < NS; ++n) k[n] = cin[n];
    } else {
#pragma unroll
        for (int n = 0; n < NS; ++n) k[n] = 0.0f;
    }
    float sig_prev = kInvLn2;  // h = ln2 * sig_prev * k  (structured path)
    float wsum = 0.0f;

    for (int64_t t0 = t_begin; t0 < t_end; t0 += kTile) {
        const int ntok = (int)min<int64_t>(kTile, t_end - t0);
        __syncthreads();  // the previous tile's B/C are no longer read
        {
            float* flat = reinterpret_cast<float*>(bc);
            for (int idx = tid; idx < 2 * NS * kTile; idx += kBlock) {
                const int which = idx / (NS * kTile);
                const int rem = idx - which * (NS * kTile);
                const int n = rem / kTile;
                const int j = rem - n * kTile;
                float v = 0.0f;
                if (n < a.N && j < ntok) {
                    const Tin* src = which ? Cg : Bg;
                    v = InTraits<Tin>::ld(src, (int64_t)n * a.L + t0 + j);
                }
                flat[(j * 2 + which) * NS + n] = v;
            }
        }
        float uu[kTile], dl[kTile], zz[kTile];
        load_row_tile<Tin>(u_row, t0, ntok, vec, uu);
        load_row_tile<Tin>(d_row, t0, ntok, vec, dl);
        if (has_z) load_row_tile<Tin>(z_row, t0, ntok, vec, zz);
        __syncthreads();

        float yv[kTile];
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            yv[j] = 0.0f;
            if (j >= ntok) continue;  // uniform across the workgroup
            const float vl = __builtin_fmaf(dl[j], kLog2e, bias_l);
            const float w = a.softplus ? softplus_log2(vl) : vl;
            if (MODE == 1) wsum += w;
            float Bn[NS], Cn[NS];
#pragma unroll
            for (int q4 = 0; q4 < NS / 4; ++q4) {
                const float4 bb = bc[j][0][q4];
                Bn[4 * q4] = bb.x; Bn[4 * q4 + 1] = bb.y; Bn[4 * q4 + 2] = bb.z; Bn[4 * q4 + 3] = bb.w;
                if (MODE == 0) {
                    const float4 cc = bc[j][1][q4];
                    Cn[4 * q4] = cc.x; Cn[4 * q4 + 1] = cc.y; Cn[4 * q4 + 2] = cc.z; Cn[4 * q4 + 3] = cc.w;
                }
            }
            float acc = 0.0f;
            if constexpr (STRUCT) {
                const float sig = w * uu[j];
                const float r = fast_exp2(w * A0);
                const bool ok = fabsf(sig) >= kSigLo && fabsf(sig) <= kSigHi;
                if (wave_all(ok)) {
                    float q = sig_prev * fast_rcp(sig) * r;
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        k[n] = __builtin_fmaf(q, k[n], Bn[n]);
                        if (MODE == 0) acc = __builtin_fmaf(Cn[n], k[n], acc);
                        q *= r;
                    }
                    sig_prev = sig;
                } else {
                    const float sig_new = ok ? sig : sig_prev;
                    const float c = sig / sig_new;
                    float q = (sig_prev / sig_new) * r;
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        k[n] = __builtin_fmaf(q, k[n], c * Bn[n]);
                        if (MODE == 0) acc = __builtin_fmaf(Cn[n], k[n], acc);
                        q *= r;
                    }
                    sig_prev = sig_new;
                }
                if (MODE == 0) {
                    float yy = __builtin_fmaf(sig_prev, acc, Dp * uu[j]);
                    yy *= has_z ? silu_scaled(zz[j], kInvLn2) : kLn2;
                    yv[j] = yy;
                }
            } else {
                const float x = (w * kLn2) * uu[j];  // Delta u
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    const float dA = fast_exp2(w * Ar[n]);
                    k[n] = __builtin_fmaf(dA, k[n], x * Bn[n]);
                    if (MODE == 0) acc = __builtin_fmaf(Cn[n], k[n], acc);
                }
                if (MODE == 0) {
                    float yy = __builtin_fmaf(Dv, uu[j], acc);
                    if (has_z) yy *= silu_scaled(zz[j], 1.0f);
                    yv[j] = yy;
                }
            }
        }
        if (MODE == 0 && active)
            store_row_tile<Tout>(reinterpret_cast<Tout*>(a.y) + row * a.L, t0, ntok, vec, yv);
    }

    // state after the chunk's last token
    const float hs = STRUCT ? kLn2 * sig_prev : 1.0f;
    if (!active) return;
    if (MODE == 1) {
        float* dst = a.ws_state + (row * a.G + g) * NS;
#pragma unroll
        for (int n = 0; n < NS; ++n) dst[n] = hs * k[n];
        a.ws_w[row * a.G + g] = wsum;
    } else if (g == a.G - 1 && a.last) {
#pragma unroll
        for (int n = 0; n < NS; ++n)
            if (n < a.N) a.last[row * a.N + n] = hs * k[n];
    }
}

// True when every state of this channel satisfies A[d,n] == fl32((n+1) A[d,0]).
__device__ __forceinline__ bool row_is_structured(const M1Args& a, int64_t dd) {
    const float A0 = a.A[dd * a.N];
    bool s = true;
    for (int n = 1; n < a.N; ++n) s = s && (a.A[dd * a.N + n] == (float)(n + 1) * A0);
    return s;
}

template <typename Tin, typename Tout, int NS, int MODE>
__global__ __launch_bounds__(kBlock) void m1_scan_kernel(M1Args a) {
    __shared__ float4 bc[kTile][2][NS / 4];
    const int64_t blocks_per_batch = (a.dim + kBlock - 1) / kBlock;
    const int b = (int)(blockIdx.x / blocks_per_batch);
    const int64_t d = (blockIdx.x - (int64_t)b * blocks_per_batch) * kBlock + threadIdx.x;
    const bool active = d < a.dim;
    const int64_t dd = active ? d : a.dim - 1;
    const int g = blockIdx.y;
    const int64_t t_begin = (int64_t)g * a.chunk;
    const int64_t t_end = min<int64_t>(a.L, t_begin + a.chunk);

    // the structured path needs every padded-in state to be a real one
    const bool structured = !a.force_general && a.N == NS &&
                            __syncthreads_and(row_is_structured(a, dd) ? 1 : 0);
    if (structured)
        scan_chunk<Tin, Tout, NS, MODE, true>(a, bc, b, dd, active, t_begin, t_end, g);
    else
        scan_chunk<Tin, Tout, NS, MODE, false>(a, bc, b, dd, active, t_begin, t_end, g);
}

// Carry pass: one thread per (row, n).  Turns the per-chunk end states b_g
// (slot g) into carries-in h_in(g) (slot g), in chunk order:
//   h_in(0) = 0,   h_in(g+1) = 2^(A[d,n] W_g) h_in(g) + b_g.
template <int NS>
__global__ __launch_bounds__(256) void m1_carry_kernel(M1Args a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t rows = a.batch * a.dim;
    if (idx >= rows * NS) return;
    const int64_t row = idx / NS;
    const int n = (int)(idx - row * NS);
    const int64_t d = row % a.dim;
    const float An = (n < a.N) ? a.A[d * a.N + n] : 0.0f;
    float h = 0.0f;
    float* st = a.ws_state + row * a.G * NS + n;
    const float* W = a.ws_w + row * a.G;
    for (int g = 0; g < a.G; ++g) {
        const float bg = (g < a.G - 1) ? st[(int64_t)g * NS] : 0.0f;
        st[(int64_t)g * NS] = h;
        if (g < a.G - 1) h = __builtin_fmaf(fast_exp2(An * W[g]), h, bg);
    }
}

template <typename Tin, typename Tout, int NS>
hipError_t launch_ns(const M1Args& a, hipStream_t stream) {
    const int64_t blocks_per_batch = (a.dim + kBlock - 1) / kBlock;
    const dim3 block(kBlock);
    if (a.G > 1) {
        const dim3 grid1((unsigned)(blocks_per_batch * a.batch), (unsigned)(a.G - 1));
        hipLaunchKernelGGL((m1_scan_kernel<Tin, Tout, NS, 1>), grid1, block, 0, stream, a);
        const int64_t threads = a.batch * a.dim * NS;
        hipLaunchKernelGGL((m1_carry_kernel<NS>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                           stream, a);
    }
    const dim3 grid0((unsigned)(blocks_per_batch * a.batch), (unsigned)a.G);
    hipLaunchKernelGGL((m1_scan_kernel<Tin, Tout, NS, 0>), grid0, block, 0, stream, a);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_dt(const M1Args& a, hipStream_t stream) {
    if (a.N <= 4) return launch_ns<Tin, Tout, 4>(a, stream);
    if (a.N <= 8) return launch_ns<Tin, Tout, 8>(a, stream);
    return launch_ns<Tin, Tout, 16>(a, stream);
}

}  // namespace

int m1_padded_states(int N) { return N <= 4 ? 4 : (N <= 8 ? 8 : 16); }

hipError_t launch_m1(const M1Args& a, int in_bf16, int out_bf16, hipStream_t stream) {
    if (in_bf16 && out_bf16) return launch_dt<uint16_t, uint16_t>(a, stream);
    if (in_bf16) return launch_dt<uint16_t, float>(a, stream);
    if (out_bf16) return launch_dt<float, uint16_t>(a, stream);
    return launch_dt<float, float>(a, stream);
}

}  // namespace selscan
