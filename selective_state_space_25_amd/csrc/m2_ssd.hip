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
// order.  The products run as v_mfma_f32_16x16x32_bf16 with fp32
// accumulation.  x, B and C are bf16 on input and enter exactly; M, S and the
// weighted x are fp32 and enter as a bf16 pair hi + lo (hi = bf16(v),
// lo = bf16(v - hi)), two MFMAs each, which keeps their relative error near
// 2^-16.  bf16 inputs, P = 64 and N in {64, 128} only; other shapes use the
// recurrent kernel.
//
// Waves 0..3 own the state: wave w holds S[:, 16w .. 16w + 16) in N / 16
// accumulator tiles and computes C S, M X and the state update for those
// columns, the state entering C S straight from its registers.  Waves 4..7
// build M, the weighted x and the decay prefix, and write y.  Every chunk
// input stays in LDS in its memory layout ([token][channel] rows): operands
// that need the other orientation are read with the transposing LDS load
// (ds_read_b64_tr_b16), which hands each lane four consecutive rows of one
// column.
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

constexpr int kQ = 64;                     // tokens per chunk
constexpr int kPd = 64;                    // headdim handled by this kernel
constexpr int kWaves = 8;                  // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kOwners = 4;                 // waves holding the state, 16 columns each
constexpr int kRowX = kPd + 8;             // padded row (elements) of x, z, weighted x
constexpr int kRowM = kQ + 8;              // padded row of M
constexpr int kRowY = kPd + 4;             // padded row (floats) of Y

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS traffic only: global loads and stores in flight
// (the next chunk's prefetch, this chunk's y) keep running across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Eight consecutive k of an MFMA operand from two 4-element pieces.
__device__ __forceinline__ bf16x8 cat(s16x4 a, s16x4 b) {
    const s16x8 r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ s16x4 ld4(const uint16_t* p) { return *reinterpret_cast<const s16x4*>(p); }

// Transposing LDS load.  Within each group of 16 lanes, lane a passes the
// address of 4 consecutive elements; lane i receives element i % 4 of the
// pieces of lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4.  With lane a
// pointing at row r0 + a / 4, columns c0 + 4 (a % 4) .. + 3 of a row-major
// matrix, lane i gets rows r0 .. r0 + 3 of column c0 + i.
__device__ __forceinline__ s16x4 ld_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p));
}

// MFMA operand with k running down a row-major matrix m (row stride `rs`):
// lane l = 16 g + i gets rows r0 + 8 g .. r0 + 8 g + 7 of column c0 + i.
__device__ __forceinline__ bf16x8 ld_col8(const uint16_t* m, int rs, int r0, int c0, int lane) {
    const int g = lane >> 4, a = lane & 15;
    const uint16_t* p = m + (r0 + 8 * g + (a >> 2)) * rs + c0 + 4 * (a & 3);
    return cat(ld_tr(p), ld_tr(p + 4 * rs));
}

// bf16 hi/lo halves of four fp32 values, packed for a 64-bit store.
__device__ __forceinline__ void split4(const float v[4], uint2& hi, uint2& lo) {
    float h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = bf16_to_f32(f32_to_bf16(v[q]));
    hi = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
    lo = make_uint2(pack_bf16x2(v[0] - h[0], v[1] - h[1]), pack_bf16x2(v[2] - h[2], v[3] - h[3]));
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One state owner's share of a chunk's inputs, fetched a chunk ahead: token
// tid / 4 and a quarter of its x, z, B and C rows.  The words are the loads'
// raw bits (past L: the last token's); they are zeroed when staged, so no use
// of them sits right behind the loads.  Only the owners load and only the
// helpers store, so neither waits on the other kind of memory operation.
template <int N>
struct ChunkRegs {
    static constexpr int kBC = N / 32;   // 16-byte pieces of a quarter row of B (and of C)
    u32x4 x[2], z[2];
    u32x4 b[kBC], c[kBC];
    uint16_t dt;                          // wave 0: Delta of token lane
};

template <int N>
struct SsdSmem {
    static constexpr int kRowN = N + 8;
    uint16_t xs[kQ][kRowX];       // x of the chunk, [s][p]
    uint16_t zs[kQ][kRowX];       // z, [t][p]
    uint16_t Bs[kQ][kRowN];       // B, [s][n]
    uint16_t Cs[kQ][kRowN];       // C, [t][n]
    uint16_t Mh[kQ][kRowM];       // M split, [t][s]
    uint16_t Ml[kQ][kRowM];
    uint16_t Wh[kQ][kRowX];       // x weighted by 2^(cum_last - cum_s) Delta_s, split, [s][p]
    uint16_t Wl[kQ][kRowX];
    float Y[kQ][kRowY];           // M X + 2^cum C S, [t][p]
    float dl[2][kQ];              // Delta, by chunk parity
    float cum[2][kQ];             // inclusive prefix of w A within the chunk
    float wts[2][kQ];             // 2^(cum_last - cum_s) Delta_s
    float ecum[2][kQ];            // 2^cum_t
    uint16_t dtraw[2][kQ];        // Delta input of the next chunk, as loaded
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per chunk (barriers between phases):
//   A  0..3     inputs into LDS in their memory layout; next chunk requested
//   B  0..3     Y = 2^cum C S for the wave's 16 columns (S from registers)
//      4..6     M: its causal 32 x 32 blocks (0,0), (1,0), (1,1), split
//   C  0..3     Y += M X, to LDS
//      4..7     the weighted x (split); silu(z) and D x silu(z) of the
//               thread's 16 outputs; wave 4: the next chunk's decay prefix
//   D  4..7     y = Y silu(z) + D x silu(z), stored
//      0..3     S = 2^cum_last S + B^T (w X); its split for the next C S
template <typename Tout, int N, bool SP>
__global__ __launch_bounds__(kThreads) void m2_ssd_kernel(M2Args a) {
    constexpr int NT = N / 16;               // 16-row state tiles per owner
    constexpr int KS = N / 32;               // k-steps over n
    constexpr int kRowN = SsdSmem<N>::kRowN;
    __shared__ __attribute__((aligned(16))) SsdSmem<N> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 15;                // MFMA column / row within a 16-tile
    const int lg = lane >> 4;                // lane group: k offset 8 lg, output rows 4 lg + q
    const bool owner = wave < kOwners;
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
    Tout* Yg = reinterpret_cast<Tout*>(a.y);

    // owners: state column p = 16 wave + li; tile j holds rows n = 16 j + 4 lg + q
    const int pcol = 16 * wave + li;
    f32x4 S[NT];
    bf16x8 Sh[KS], Sl[KS];   // the state split as C S operands (k-step ks: tiles 2 ks, 2 ks + 1)
    auto split_state = [&]() {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = S[2 * ks + (j >> 2)][j & 3];
                const __bf16 hv = (__bf16)v;
                Sh[ks][j] = hv;
                Sl[ks][j] = (__bf16)(v - (float)hv);
            }
        }
    };
    if (owner) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                S[j][q] = a.h0 ? a.h0[(bh * kPd + pcol) * N + 16 * j + 4 * lg + q] : 0.0f;
        split_state();
    }

    const int64_t nch = (L + kQ - 1) / kQ;
    constexpr int NBC = ChunkRegs<N>::kBC;
    const int rt = tid >> 2, rq = tid & 3;   // owners: token, quarter row
    // Loads are unconditional, from the last token's addresses past L (and
    // from x when there is no z).
    auto fetch = [&](int64_t t0, ChunkRegs<N>& r) {
        // Delta first: wave 0 hands it on through LDS before the rest lands
        if (wave == 0) r.dt = DT[(b * L + (t0 + lane < L ? t0 + lane : L - 1)) * H + h];
        const int64_t tt = t0 + rt < L ? t0 + rt : L - 1;
        const u32x4* xp = reinterpret_cast<const u32x4*>(X + ((b * L + tt) * H + h) * kPd + 16 * rq);
        const u32x4* zp = reinterpret_cast<const u32x4*>((Z ? Z : X) + ((b * L + tt) * H + h) * kPd + 16 * rq);
        const int64_t bo = ((b * L + tt) * G + grp) * N + (N / 4) * rq;
        r.x[0] = xp[0];
        r.x[1] = xp[1];
        r.z[0] = zp[0];
        r.z[1] = zp[1];
#pragma unroll
        for (int q = 0; q < NBC; ++q) {
            r.b[q] = reinterpret_cast<const u32x4*>(Bg + bo)[q];
            r.c[q] = reinterpret_cast<const u32x4*>(Cg + bo)[q];
        }
    };
    // Delta, the in-chunk prefix of the log2 decay and the per-token factors
    // of the chunk at t0 (tokens past L: Delta 0, decay 1, no input)
    auto prefix = [&](int64_t t0, int buf) {
        float wv = 0.0f;
        if (t0 + lane < L) {
            const float vl = __builtin_fmaf(bf16_to_f32(sm.dtraw[buf][lane]), kLog2e, bias_l);
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
        sm.dl[buf][lane] = dlv;
        sm.cum[buf][lane] = cs;
        sm.ecum[buf][lane] = fast_exp2(cs);
        sm.wts[buf][lane] = fast_exp2(last - cs) * dlv;
    };

    ChunkRegs<N> cr;
    if (owner) {
        fetch(0, cr);
        if (wave == 0) sm.dtraw[0][lane] = cr.dt;
    }
    lds_barrier();
    if (wave == kOwners) prefix(0, 0);

    // helpers: the thread's token and 16 outputs of the epilogue (and of the
    // weighted x): t = ht / 4, p = 16 (ht % 4) ..
    const int ht = tid - kOwners * 64;
    const int et = ht >> 2, ep0 = (ht & 3) * 16;
    float eg[16], edg[16];   // silu(z) and D x silu(z), from phase C to D

    for (int64_t c = 0; c < nch; ++c) {
        const int64_t t0 = c * kQ;
        const int cb = (int)(c & 1);
        if (owner) {
            // ---- A: stage this chunk in its memory layout; request the next ----
            const bool part = t0 + kQ > L;   // a partial last chunk: zero past L
            const unsigned keep = (!part || t0 + rt < L) ? ~0u : 0u;
            const unsigned keepz = Z ? keep : 0u;
            u32x4* xd = reinterpret_cast<u32x4*>(&sm.xs[rt][16 * rq]);
            u32x4* zd = reinterpret_cast<u32x4*>(&sm.zs[rt][16 * rq]);
            xd[0] = cr.x[0] & keep;
            xd[1] = cr.x[1] & keep;
            zd[0] = cr.z[0] & keepz;
            zd[1] = cr.z[1] & keepz;
            u32x4* bd = reinterpret_cast<u32x4*>(&sm.Bs[rt][(N / 4) * rq]);
            u32x4* cd = reinterpret_cast<u32x4*>(&sm.Cs[rt][(N / 4) * rq]);
#pragma unroll
            for (int q = 0; q < NBC; ++q) {
                bd[q] = cr.b[q] & keep;
                cd[q] = cr.c[q] & keep;
            }
            if (c + 1 < nch) fetch(t0 + kQ, cr);
        }
        lds_barrier();

        f32x4 Yacc[4];
        if (owner) {
            // ---- B (owners): Y = 2^cum C S, the state from registers ----------
            // k-step ks pairs state tiles 2 ks and 2 ks + 1, whose rows
            // 4 lg .. 4 lg + 3 this lane holds: the C operand takes columns
            // 32 ks + 4 lg .. + 3 and 32 ks + 16 + 4 lg .. + 3 in that order
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                Yacc[tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                const uint16_t* crow = &sm.Cs[16 * tb + li][4 * lg];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 cv = cat(ld4(crow + 32 * ks), ld4(crow + 32 * ks + 16));
                    Yacc[tb] = mfma(cv, Sh[ks], Yacc[tb]);
                    Yacc[tb] = mfma(cv, Sl[ks], Yacc[tb]);
                }
                Yacc[tb] *= *reinterpret_cast<const f32x4*>(&sm.ecum[cb][16 * tb + 4 * lg]);
            }
            // the next chunk's Delta inputs for the prefix wave
            if (wave == 0 && c + 1 < nch) sm.dtraw[cb ^ 1][lane] = cr.dt;
        } else if (wave < kOwners + 3) {
            // ---- B (helpers): a causal 32 x 32 block of M ---------------------
            // block (t, s) = (0, 0), (1, 0), (1, 1) as M^T = B C^T: lane
            // column t = 32 tb + lane % 32, rows s = 32 sb + 8 r + 4 h + q
            const int hw = wave - kOwners;
            const int tb = hw == 0 ? 0 : 1, sb = hw == 2 ? 1 : 0;
            const int l32 = lane & 31, h = lane >> 5;
            f32x16 g = {};
#pragma unroll
            for (int kk = 0; kk < N / 16; ++kk)
                g = mfma32(ld8(&sm.Bs[32 * sb + l32][16 * kk + 8 * h]), ld8(&sm.Cs[32 * tb + l32][16 * kk + 8 * h]), g);
            const int t = 32 * tb + l32;
            const float ct = sm.cum[cb][t];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s0 = 32 * sb + 8 * r + 4 * h;
                const f32x4 cs = *reinterpret_cast<const f32x4*>(&sm.cum[cb][s0]);
                const f32x4 ds = *reinterpret_cast<const f32x4*>(&sm.dl[cb][s0]);
                float m[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    m[q] = (s0 + q <= t) ? g[4 * r + q] * fast_exp2(ct - cs[q]) * ds[q] : 0.0f;
                uint2 mh, ml;
                split4(m, mh, ml);
                *reinterpret_cast<uint2*>(&sm.Mh[t][s0]) = mh;
                *reinterpret_cast<uint2*>(&sm.Ml[t][s0]) = ml;
            }
        }
        lds_barrier();

        if (owner) {
            // ---- C (owners): Y += M X over the causal k-steps; Y to LDS -------
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
                for (int ks = 0; ks <= (tb >> 1); ++ks) {
                    const bf16x8 xv = ld_col8(&sm.xs[0][0], kRowX, 32 * ks, 16 * wave, lane);
                    Yacc[tb] = mfma(ld8(&sm.Mh[16 * tb + li][32 * ks + 8 * lg]), xv, Yacc[tb]);
                    Yacc[tb] = mfma(ld8(&sm.Ml[16 * tb + li][32 * ks + 8 * lg]), xv, Yacc[tb]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) sm.Y[16 * tb + 4 * lg + q][pcol] = Yacc[tb][q];
            }
        } else {
            // ---- C (helpers): weighted x; the gate of the thread's outputs ----
            const float wv = sm.wts[cb][et];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const bf16x8 xv = ld8(&sm.xs[et][ep0 + 8 * half]);
                const bf16x8 zv = ld8(&sm.zs[et][ep0 + 8 * half]);
                bf16x8 xh, xl;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float x = (float)xv[j];
                    const float v = x * wv;
                    const __bf16 vh = (__bf16)v;
                    xh[j] = vh;
                    xl[j] = (__bf16)(v - (float)vh);
                    const float gz = Z ? silu_scaled((float)zv[j], 1.0f) : 1.0f;
                    eg[8 * half + j] = gz;
                    edg[8 * half + j] = Dh * x * gz;
                }
                *reinterpret_cast<bf16x8*>(&sm.Wh[et][ep0 + 8 * half]) = xh;
                *reinterpret_cast<bf16x8*>(&sm.Wl[et][ep0 + 8 * half]) = xl;
            }
            if (wave == kOwners && c + 1 < nch) prefix(t0 + kQ, cb ^ 1);
        }
        lds_barrier();

        if (!owner) {
            // ---- D (helpers): y = Y silu(z) + D x silu(z), stored --------------
            if (t0 + et < L) {
                float yv[16];
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const f32x4 yy = *reinterpret_cast<const f32x4*>(&sm.Y[et][ep0 + 4 * j4]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) yv[4 * j4 + q] = __builtin_fmaf(yy[q], eg[4 * j4 + q], edg[4 * j4 + q]);
                }
                Tout* dst = Yg + ((b * L + t0 + et) * H + h) * kPd + ep0;
                if constexpr (sizeof(Tout) == 4) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        reinterpret_cast<float4*>(dst)[q] =
                            make_float4(yv[4 * q], yv[4 * q + 1], yv[4 * q + 2], yv[4 * q + 3]);
                } else {
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        reinterpret_cast<uint4*>(dst)[q] =
                            make_uint4(pack_bf16x2(yv[8 * q], yv[8 * q + 1]), pack_bf16x2(yv[8 * q + 2], yv[8 * q + 3]),
                                       pack_bf16x2(yv[8 * q + 4], yv[8 * q + 5]),
                                       pack_bf16x2(yv[8 * q + 6], yv[8 * q + 7]));
                }
            }
        } else {
            // ---- D (owners): S = 2^cum_last S + B^T (w X) ---------------------
            const float dec = sm.ecum[cb][kQ - 1];
            bf16x8 wh[2], wl[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                wh[ks] = ld_col8(&sm.Wh[0][0], kRowX, 32 * ks, 16 * wave, lane);
                wl[ks] = ld_col8(&sm.Wl[0][0], kRowX, 32 * ks, 16 * wave, lane);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                S[j] *= dec;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    // B^T operand: row n = 16 j + li, k = s
                    const bf16x8 bt = ld_col8(&sm.Bs[0][0], kRowN, 32 * ks, 16 * j, lane);
                    S[j] = mfma(bt, wh[ks], S[j]);
                    S[j] = mfma(bt, wl[ks], S[j]);
                }
            }
            split_state();
        }
        lds_barrier();
    }

    if (a.last && owner) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) a.last[(bh * kPd + pcol) * N + 16 * j + 4 * lg + q] = S[j][q];
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
