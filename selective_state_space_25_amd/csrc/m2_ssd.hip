// m2_ssd.hip -- Mamba-2 scan in chunked (state-space-duality) form on MFMA.
//
// The Mamba README's Mamba-2 section names the SSD formulation: with a scalar
// decay per head the recurrence of one head over a chunk of Q tokens is a
// masked matrix product plus a low-rank carry.  In log2 units, with
// w_t = Delta_t / ln2, l_t = w_t A_h and cum_t = sum_{s <= t} l_s inside the
// chunk (S the [N, P] state entering the chunk, X the chunk's x of the head):
//
//   M[t, s] = (C_t . B_s) 2^(cum_t - cum_s) Delta_s        (s <= t, else 0)
//   Y       = M X + diag(2^cum_t) C S
//   S'      = 2^cum_last S + B^T diag(2^(cum_last - cum_s) Delta_s) X
//
// which is the plain recurrence h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t,
// y_t = C_t h_t, regrouped (the contractions over n and s are exact sums).
// y then gets D x and the silu(z) gate as in the recurrent kernel.
//
// One workgroup (8 waves) owns one (batch, head) and walks its chunks in
// order, the state in MFMA accumulators.  The products run as
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  x, B and C are bf16 on
// input and enter exactly; M, S and the weighted X are fp32 and enter as a
// bf16 pair hi + lo (hi = bf16(v), lo = bf16(v - hi)), two MFMAs each, which
// keeps their relative error near 2^-16.  bf16 inputs, P = 64 and N in
// {64, 128} only; other shapes use the recurrent kernel.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQ = 64;    // tokens per chunk
constexpr int kPd = 64;   // headdim handled by this kernel
constexpr int kPadQ = kQ + 8;

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ uint16_t bf16_bits(float v) { return f32_to_bf16(v); }

// v = hi + lo with both halves bf16
__device__ __forceinline__ void split(float v, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16(v);
    lo = f32_to_bf16(v - bf16_to_f32(hi));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS traffic only: global loads and stores in flight
// (the next chunk's prefetch, this chunk's y) keep running across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

constexpr int kWaves = 8;                  // waves per workgroup
constexpr int kThreads = 64 * kWaves;

// One thread's share of a chunk's inputs, fetched a chunk ahead: token
// tid / 8, eight channels of x and z and N / 8 states of B and C.
template <int N>
struct ChunkRegs {
    static constexpr int PER = N / 8;
    uint4 x, z;
    uint4 b[PER / 8], c[PER / 8];
    uint16_t dt;
};

// Row index of accumulator register i (= 4 r + q) of this lane inside a
// 32 x 32 block; the column is lane % 32.
__device__ __forceinline__ int acc_row(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

template <int N>
struct SsdSmem {
    static constexpr int kPadN = N + 8;
    uint16_t xT[kPd][kPadQ];      // x of the chunk, [p][s]
    uint16_t zs[kQ][kPd + 8];     // z of the chunk, [t][p]
    uint16_t Cs[kQ][kPadN];       // C, [t][n]
    uint16_t Bs[kQ][kPadN];       // B, [s][n]
    uint16_t BT[N][kPadQ];        // B, [n][s]
    uint16_t Mh[kQ][kPadQ];       // M split, [t][s]
    uint16_t Ml[kQ][kPadQ];
    uint16_t STh[kPd][kPadN];     // state entering the chunk, split, [p][n]
    uint16_t STl[kPd][kPadN];
    uint16_t XWh[kPd][kPadQ];     // x weighted by 2^(cum_last - cum_s) Delta_s, split, [p][s]
    uint16_t XWl[kPd][kPadQ];
    float yoff[4][16][64];        // C S of each 32 x 32 output block, [block][register][lane]
    float dl[kQ];                 // Delta
    float cum[kQ];                // inclusive prefix of w A within the chunk
    float wts[kQ];                // 2^(cum_last - cum_s) Delta_s
};

// Eight waves per (batch, head).  Per chunk:
//   stage   all      inputs into LDS (x also transposed, B also as [n][s]),
//                    the entering state as split bf16; wave 0: Delta, the
//                    decay prefix and the state-update weights
//   M       0..2     the three causal 32 x 32 blocks of (C B^T) o decay
//           4..7     the weighted x, split (16 tokens each)
//   Y       0..3     M X of output block (t, p) = (w / 2, w % 2)
//           4..7     C S of the same block, to LDS
//   out     0..3     Y = M X + 2^cum C S + D x, gate, store
//   S       w < 2N/32  state block (n, p) = (w / 2, w % 2):
//                    S = 2^cum_last S + B^T (w X)
template <typename Tout, int N, bool SP>
__global__ __launch_bounds__(kThreads) void m2_ssd_kernel(M2Args a) {
    constexpr int NB = N / 32;               // row blocks of the state
    __shared__ __attribute__((aligned(16))) SsdSmem<N> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int col = lane & 31;
    const int khalf = (lane >> 5) * 8;       // k offset of this lane inside a 16-wide step
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / a.H;
    const int64_t h = bh - b * a.H;
    const int64_t grp = h / (a.H / a.G);
    const int64_t L = a.L;
    const int64_t H = a.H, G = a.G;
    const float Ah = a.A[h];
    const float bias_l = (a.dt_bias ? a.dt_bias[h] : 0.0f) * kLog2e;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* DT = reinterpret_cast<const uint16_t*>(a.dt);
    const uint16_t* Bg = reinterpret_cast<const uint16_t*>(a.B);
    const uint16_t* Cg = reinterpret_cast<const uint16_t*>(a.C);
    const uint16_t* Z = reinterpret_cast<const uint16_t*>(a.z);
    Tout* Y = reinterpret_cast<Tout*>(a.y);

    // this wave's state block (n, p), if any
    const bool owns = wave < 2 * NB;
    const int s_ni = wave >> 1, s_pj = wave & 1;
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int n = 32 * s_ni + acc_row(i, lane);
        const int p = 32 * s_pj + col;
        S[i] = (owns && a.h0) ? a.h0[(bh * kPd + p) * N + n] : 0.0f;
    }

    const int64_t nch = (L + kQ - 1) / kQ;
    constexpr int PER = N / 8;
    const int rt = tid >> 3, rp0 = (tid & 7) * 8, rn0 = (tid & 7) * PER;
    auto fetch = [&](int64_t t0, ChunkRegs<N>& r) {
        const bool in = t0 + rt < L;
        const uint4 zero = make_uint4(0, 0, 0, 0);
        const int64_t xo = ((b * L + t0 + rt) * H + h) * kPd + rp0;
        const int64_t bo = ((b * L + t0 + rt) * G + grp) * N + rn0;
        r.x = in ? *reinterpret_cast<const uint4*>(X + xo) : zero;
        r.z = (in && Z) ? *reinterpret_cast<const uint4*>(Z + xo) : zero;
#pragma unroll
        for (int q = 0; q < PER / 8; ++q) {
            r.b[q] = in ? reinterpret_cast<const uint4*>(Bg + bo)[q] : zero;
            r.c[q] = in ? reinterpret_cast<const uint4*>(Cg + bo)[q] : zero;
        }
        r.dt = (wave == 0 && t0 + lane < L) ? DT[(b * L + t0 + lane) * H + h] : (uint16_t)0;
    };
    ChunkRegs<N> cr;
    fetch(0, cr);
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t t0 = c * kQ;
        // ---- stage: the entering state, split, [p][n]; this chunk's inputs
        if (owns) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int n = 32 * s_ni + acc_row(i, lane);
                const int p = 32 * s_pj + col;
                uint16_t hi, lo;
                split(S[i], hi, lo);
                sm.STh[p][n] = hi;
                sm.STl[p][n] = lo;
            }
        }
        {
            const uint32_t w[4] = {cr.x.x, cr.x.y, cr.x.z, cr.x.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sm.xT[rp0 + 2 * j][rt] = (uint16_t)(w[j] & 0xffffu);
                sm.xT[rp0 + 2 * j + 1][rt] = (uint16_t)(w[j] >> 16);
            }
            *reinterpret_cast<uint4*>(&sm.zs[rt][rp0]) = cr.z;
#pragma unroll
            for (int q = 0; q < PER / 8; ++q) {
                *reinterpret_cast<uint4*>(&sm.Bs[rt][rn0 + 8 * q]) = cr.b[q];
                *reinterpret_cast<uint4*>(&sm.Cs[rt][rn0 + 8 * q]) = cr.c[q];
                const uint32_t wb[4] = {cr.b[q].x, cr.b[q].y, cr.b[q].z, cr.b[q].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sm.BT[rn0 + 8 * q + 2 * j][rt] = (uint16_t)(wb[j] & 0xffffu);
                    sm.BT[rn0 + 8 * q + 2 * j + 1][rt] = (uint16_t)(wb[j] >> 16);
                }
            }
        }
        if (wave == 0) {
            // Delta and the in-chunk prefix of the log2 decay (tokens past L:
            // Delta 0, decay 1, no input)
            const int t = lane;
            float wv = 0.0f;
            if (t0 + t < L) {
                const float vl = __builtin_fmaf(bf16_to_f32(cr.dt), kLog2e, bias_l);
                wv = SP ? softplus_log2(vl) : vl;
            }
            float cs = wv * Ah;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float up = __shfl_up(cs, o, 64);
                if (lane >= o) cs += up;
            }
            const float last = __shfl(cs, 63, 64);
            const float dlv = wv * kLn2;
            sm.dl[t] = dlv;
            sm.cum[t] = cs;
            sm.wts[t] = fast_exp2(last - cs) * dlv;
        }
        if (c + 1 < nch) fetch(t0 + kQ, cr);
        lds_barrier();

        // ---- M = (C B^T) o decay: blocks (0,0), (1,0), (1,1); weighted x --
        if (wave < 3) {
            const int ti = wave == 0 ? 0 : 1;
            const int si = wave == 2 ? 1 : 0;
            f32x16 g = {};
#pragma unroll
            for (int kk = 0; kk < N / 16; ++kk) {
                const bf16x8 av = ld8(&sm.Cs[32 * ti + col][16 * kk + khalf]);
                const bf16x8 bv = ld8(&sm.Bs[32 * si + col][16 * kk + khalf]);
                g = mfma(av, bv, g);
            }
            const int s = 32 * si + col;
            const float cs = sm.cum[s];
            const float ds = sm.dl[s];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = 32 * ti + acc_row(i, lane);
                const float m = t >= s ? g[i] * fast_exp2(sm.cum[t] - cs) * ds : 0.0f;
                uint16_t hi, lo;
                split(m, hi, lo);
                sm.Mh[t][s] = hi;
                sm.Ml[t][s] = lo;
            }
        } else if (wave >= 4) {
            const int p = lane;
#pragma unroll
            for (int s8 = 0; s8 < 2; ++s8) {
                const int s0 = 16 * (wave - 4) + 8 * s8;
                const bf16x8 xv = ld8(&sm.xT[p][s0]);
                bf16x8 xh, xl;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float v = (float)xv[j] * sm.wts[s0 + j];
                    const __bf16 vh = (__bf16)v;
                    xh[j] = vh;
                    xl[j] = (__bf16)(v - (float)vh);
                }
                *reinterpret_cast<bf16x8*>(&sm.XWh[p][s0]) = xh;
                *reinterpret_cast<bf16x8*>(&sm.XWl[p][s0]) = xl;
            }
        }
        lds_barrier();

        // ---- Y: M X on waves 0..3, C S (to LDS) on waves 4..7 ------------
        const int yb = wave & 3;
        const int ti = yb >> 1, pj = yb & 1;
        f32x16 yi = {};
        if (wave < 4) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk >= 2 * (ti + 1)) break;   // causal: s < 32 (ti + 1)
                const bf16x8 xv = ld8(&sm.xT[32 * pj + col][16 * kk + khalf]);
                yi = mfma(ld8(&sm.Mh[32 * ti + col][16 * kk + khalf]), xv, yi);
                yi = mfma(ld8(&sm.Ml[32 * ti + col][16 * kk + khalf]), xv, yi);
            }
        } else {
            f32x16 yc = {};
#pragma unroll
            for (int kk = 0; kk < N / 16; ++kk) {
                const bf16x8 cv = ld8(&sm.Cs[32 * ti + col][16 * kk + khalf]);
                yc = mfma(cv, ld8(&sm.STh[32 * pj + col][16 * kk + khalf]), yc);
                yc = mfma(cv, ld8(&sm.STl[32 * pj + col][16 * kk + khalf]), yc);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.yoff[yb][i][lane] = yc[i];
        }
        lds_barrier();

        // ---- out: Y = M X + 2^cum C S + D x, the gate, the store -----------
        if (wave < 4) {
            const int p = 32 * pj + col;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = 32 * ti + acc_row(i, lane);
                if (t0 + t >= L) continue;
                const float xv = bf16_to_f32(sm.xT[p][t]);
                float yv = __builtin_fmaf(fast_exp2(sm.cum[t]), sm.yoff[yb][i][lane], yi[i]);
                yv = __builtin_fmaf(Dh, xv, yv);
                const int64_t idx = ((b * L + t0 + t) * H + h) * kPd + p;
                if (Z) yv *= silu_scaled(bf16_to_f32(sm.zs[t][p]), 1.0f);
                if constexpr (sizeof(Tout) == 4)
                    Y[idx] = yv;
                else
                    Y[idx] = f32_to_bf16(yv);
            }
        }

        // ---- S = 2^cum_last S + B^T diag(wts) X ---------------------------
        if (owns) {
            const float dec = fast_exp2(sm.cum[kQ - 1]);
#pragma unroll
            for (int i = 0; i < 16; ++i) S[i] *= dec;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 bv = ld8(&sm.BT[32 * s_ni + col][16 * kk + khalf]);
                const int p = 32 * s_pj + col;
                S = mfma(bv, ld8(&sm.XWh[p][16 * kk + khalf]), S);
                S = mfma(bv, ld8(&sm.XWl[p][16 * kk + khalf]), S);
            }
        }
        lds_barrier();
    }

    if (a.last && owns) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int n = 32 * s_ni + acc_row(i, lane);
            const int p = 32 * s_pj + col;
            a.last[(bh * kPd + p) * N + n] = S[i];
        }
    }
}

template <typename Tout, int N>
hipError_t launch_n(const M2Args& a, hipStream_t stream) {
    const unsigned blocks = (unsigned)(a.batch * a.H);
    KTime kt("m2_ssd", stream);
    if (a.softplus)
        hipLaunchKernelGGL((m2_ssd_kernel<Tout, N, true>), dim3(blocks), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((m2_ssd_kernel<Tout, N, false>), dim3(blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool m2_ssd_supported(const M2Args& a, int in_bf16) {
    return in_bf16 && a.P == kPd && (a.N == 64 || a.N == 128) && a.batch * a.H < 0x7fffffff;
}

hipError_t launch_m2_ssd(const M2Args& a, int out_bf16, hipStream_t stream) {
    if (a.N == 128) return out_bf16 ? launch_n<uint16_t, 128>(a, stream) : launch_n<float, 128>(a, stream);
    return out_bf16 ? launch_n<uint16_t, 64>(a, stream) : launch_n<float, 64>(a, stream);
}

}  // namespace selscan
