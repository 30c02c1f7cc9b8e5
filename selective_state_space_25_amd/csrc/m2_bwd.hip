// m2_bwd.hip -- gradients of the Mamba-2 (multi-head) selective scan, gfx950.
//
// The forward is the Mamba-2 layer of the Mamba README (section "Mamba-2";
// skill page "model-architecture-mamba": heads, headdim, d_state, groups):
// per (batch b, head h, channel p) the Mamba-1 recurrence of section 2.2 of
// the "Understanding Mamba and Selective State Space Models (SSMs)" blog
// with one scalar decay per (token, head) and B, C shared by the heads of a
// group g = h / (H / G):
//
//   Delta_t = softplus(dt_t + bias_h),  a_t = exp(Delta_t A_h)
//   h_t[n]  = a_t h_{t-1}[n] + Delta_t x_t[p] B_t[n]
//   out_t   = (sum_n C_t[n] h_t[n] + D_h x_t[p]) silu(z_t[p])
//
// Reverse mode, with dy_t = dout_t silu(z_t) and the state's adjoint
// lam_t[n] = dy_t C_t[n] + a_{t+1} lam_{t+1}[n] running backward in time:
//
//   dx_t[p]   = Delta_t sum_n lam_t[n] B_t[n] + D_h dy_t
//   dDelta_t  = sum_{p,n} lam_t (x_t B_t + A_h a_t h_{t-1})
//   dA_h      = sum_t Delta_t a_t sum_{p,n} lam_t h_{t-1}
//   dB_t[n]   = sum_{h in g, p} lam_t[n] Delta_t x_t[p]
//   dC_t[n]   = sum_{h in g, p} dy_t[p] h_t[n]
//   dz_t      = dout_t y_t silu'(z_t),  dD_h = sum dy x,  dh0 = a_0 lam_0
//
// Work layout: one workgroup per (batch, head), N / 16 waves; wave w holds
// states n = 16 w .. 16 w + 15 of all 64 channels, lane = channel p.
//  - checkpoint pass: the forward recurrence, storing every 8th state (the
//    state entering each 8-token tile) to the workspace;
//  - adjoint pass: tiles from the last, each recomputing its 8 tokens'
//    states from the tile's checkpoint into registers, then running the
//    adjoint back through them.  Sums over n (dx, dDelta) go over the 16
//    states in a lane and the waves through LDS; sums over p (dB, dC) are
//    reduced across the lanes with permlane swaps and DPP row sums and
//    stored per head;
//  - reduce: dB, dC over the heads of a group, dA, dD, dbias over batches,
//    in a fixed order (results are reproducible bit for bit).
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

constexpr int kT2 = 8;   // tokens per tile (and per checkpoint)
constexpr int kP = 64;   // headdim = lanes

template <typename T> __device__ __forceinline__ float ldf(const T* p, int64_t i);
template <> __device__ __forceinline__ float ldf<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kRor4 = 0x124, kRor8 = 0x128, kQuadX1 = 0xB1, kQuadX2 = 0x4E;

// sum over the 16 lanes of a DPP row, in every lane of the row
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<kRor8>(v);
    v += dpp<kRor4>(v);
    v += dpp<kQuadX2>(v);
    return v + dpp<kQuadX1>(v);
}

// sum over the 64 lanes of the wave, in every lane
__device__ __forceinline__ float wave_sum(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    return row_sum(v);
}

// Sums over the 64 lanes of 32 per-lane values (v[0..15], then u[0..15]),
// reduce-scattered: each exchange hands half of a lane's values to the
// partner that keeps the other half and adds what it receives.  permlane32
// swaps pair value m with m + 16 (lanes 0..31 keep v, 32..63 keep u),
// permlane16 swaps pair m with m + 8, then within each 16-lane row the
// partners lane ^ 8 (row rotation by 8), the mirrored lane of the 8-lane
// half (bit 2 differs), lane ^ 2 and lane ^ 1 (quad permutes).  Lane l ends
// with the sum of value 8 (l >> 4) + 4 b3 + 2 b2 + b1 (b = bits of l; 0..15
// from v, 16..31 from u), in lanes l and l ^ 1.
constexpr int kHalfMirror = 0x141;
__device__ __forceinline__ float pick(bool hi, float a, float b) { return hi ? b : a; }
__device__ __forceinline__ float reduce32(const float* v, const float* u) {
    float x[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[m]), __float_as_uint(u[m]), false, false);
        x[m] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
    float y[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[m]), __float_as_uint(x[m + 8]), false, false);
        y[m] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
    const int l = threadIdx.x & 63;
    const bool b3 = l & 8, b2 = l & 4, b1 = l & 2;
    float z[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) z[m] = pick(b3, y[m], y[m + 4]) + dpp<kRor8>(pick(b3, y[m + 4], y[m]));
    float w[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) w[m] = pick(b2, z[m], z[m + 2]) + dpp<kHalfMirror>(pick(b2, z[m + 2], z[m]));
    const float r = pick(b1, w[0], w[1]) + dpp<kQuadX2>(pick(b1, w[1], w[0]));
    return r + dpp<kQuadX1>(r);
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Delta / ln2 of a token (log2 units) and the softplus derivative sigmoid(v).
template <bool SP>
__device__ __forceinline__ float w_of(float v, float& deriv) {
    if (!SP) {
        deriv = 1.0f;
        return v * kLog2e;
    }
    const float e = fast_exp2(-fabsf(v) * kLog2e);   // exp(-|v|)
    const float r = fast_rcp(1.0f + e);
    deriv = v >= 0.0f ? r : e * r;
    return softplus_log2(v * kLog2e);
}

// Delta, a = exp(Delta A) and the softplus derivative of one token from its
// raw dt (tokens past L: Delta = 0, a = 1, an identity step).
template <bool SP>
__device__ __forceinline__ void tok_consts(float dtv, bool ok, float Ah, float biash, float& dl, float& av,
                                           float& dv) {
    dl = 0.0f;
    av = 1.0f;
    dv = 0.0f;
    if (ok) {
        const float w = w_of<SP>(dtv + biash, dv);
        dl = w * kLn2;
        av = fast_exp2(w * Ah);
    }
}

// One tile's global inputs held in registers while the tile before it is
// computed: this thread's two of the tile's 8 x N B (and C) values, the raw
// dt of its tokens, and x (dout, z) of its (token, channel) pairs.  Thread
// `tid` takes B/C elements e = tid and tid + 64 NW of the tile (token e / N,
// state e % N) and pairs (w + m NW, lane).
template <int NW>
struct TileRegs {
    static constexpr int kPer = (kT2 + NW - 1) / NW;
    float b[2], c[2];
    float dt[kPer], x[kPer], dout[kPer], z[kPer];
};

template <typename Tin, typename Tout, int NW, bool BWD>
__device__ __forceinline__ void load_tile(const M2BwdArgs& a, int64_t b, int64_t h, int64_t g, int64_t t0,
                                          TileRegs<NW>& r) {
    constexpr int N = 16 * NW;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const Tin* Bp = reinterpret_cast<const Tin*>(a.B);
    const Tin* Cp = reinterpret_cast<const Tin*>(a.C);
    const Tin* X = reinterpret_cast<const Tin*>(a.x);
    const Tin* DT = reinterpret_cast<const Tin*>(a.dt);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int e = tid + q * 64 * NW;
        const int j = e / N, n = e - j * N;
        const int64_t t = t0 + j;
        const int64_t i = ((b * a.L + t) * a.G + g) * N + n;
        const bool ok = t < a.L;
        r.b[q] = ok ? ldf(Bp, i) : 0.0f;
        if (BWD) r.c[q] = ok ? ldf(Cp, i) : 0.0f;
    }
#pragma unroll
    for (int m = 0; m < TileRegs<NW>::kPer; ++m) {
        const int j = w + m * NW;
        const int64_t t = t0 + j;
        const bool ok = j < kT2 && t < a.L;
        const int64_t e = ((b * a.L + t) * a.H + h) * kP + lane;
        r.dt[m] = ok ? ldf(DT, (b * a.L + t) * a.H + h) : 0.0f;
        r.x[m] = ok ? ldf(X, e) : 0.0f;
        if (BWD) {
            r.dout[m] = ok ? ldf(reinterpret_cast<const Tout*>(a.dout), e) : 0.0f;
            r.z[m] = (ok && a.z) ? ldf(reinterpret_cast<const Tin*>(a.z), e) : 0.0f;
        }
    }
}

// ---------------- checkpoint pass -------------------------------------------
template <typename Tin, int NW, bool SP>
__global__ __launch_bounds__(64 * NW) void m2_bwd_ck_kernel(M2BwdArgs a) {
    constexpr int N = 16 * NW;
    constexpr int kPer = TileRegs<NW>::kPer;
    __shared__ alignas(16) float Bs[2][kT2][N];
    __shared__ float xws[2][kT2][kP], Aa[2][kT2];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int64_t bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
    const float Ah = a.A[h], biash = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const int64_t ntiles = (a.L + kT2 - 1) / kT2;
    float hs[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) hs[i] = a.h0 ? a.h0[(bh * kP + lane) * N + 16 * w + i] : 0.0f;
    // a tile's inputs into LDS buffer `buf`: B, a per token, Delta x per pair
    auto put = [&](const TileRegs<NW>& r, int64_t t0, int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) (&Bs[buf][0][0])[tid + q * 64 * NW] = r.b[q];
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int j = w + m * NW;
            if (j < kT2) {
                float dl, av, dv;
                tok_consts<SP>(r.dt[m], t0 + j < a.L, Ah, biash, dl, av, dv);
                xws[buf][j][lane] = dl * r.x[m];
                if (lane == 0) Aa[buf][j] = av;
            }
        }
    };
    // two register sets, each loaded two tiles ahead of its use: the
    // tile's arithmetic alone (8 tokens) is shorter than a load's latency
    TileRegs<NW> ra, rb;
    load_tile<Tin, Tin, NW, false>(a, b, h, g, 0, ra);
    if (ntiles > 1) load_tile<Tin, Tin, NW, false>(a, b, h, g, kT2, rb);
    put(ra, 0, 0);
    lds_barrier();
    auto step = [&](int64_t k, TileRegs<NW>& mine, TileRegs<NW>& other) {
        const int buf = (int)(k & 1);
        if (k + 2 < ntiles) load_tile<Tin, Tin, NW, false>(a, b, h, g, (k + 2) * kT2, mine);
        // checkpoint record of (tile, wave): piece q of every lane's 16 states
        // together, so that each store covers 1 KB of consecutive bytes
        {
            float4* dst = reinterpret_cast<float4*>(a.ck + ((bh * ntiles + k) * NW + w) * (kP * 16)) + lane;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dst[64 * q] = make_float4(hs[4 * q], hs[4 * q + 1], hs[4 * q + 2], hs[4 * q + 3]);
        }
#pragma unroll
        for (int j = 0; j < kT2; ++j) {
            const float xw = xws[buf][j][lane], av = Aa[buf][j];
            const float4* br = reinterpret_cast<const float4*>(&Bs[buf][j][16 * w]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 bb = br[q];
                hs[4 * q] = __builtin_fmaf(av, hs[4 * q], xw * bb.x);
                hs[4 * q + 1] = __builtin_fmaf(av, hs[4 * q + 1], xw * bb.y);
                hs[4 * q + 2] = __builtin_fmaf(av, hs[4 * q + 2], xw * bb.z);
                hs[4 * q + 3] = __builtin_fmaf(av, hs[4 * q + 3], xw * bb.w);
            }
        }
        // buffer buf ^ 1 was last read in iteration k - 1, before its barrier
        if (k + 1 < ntiles) put(other, (k + 1) * kT2, buf ^ 1);
        lds_barrier();
    };
    for (int64_t k = 0; k < ntiles; k += 2) {
        step(k, ra, rb);          // tile k: ra (tile k's data) is free for tile k + 2
        if (k + 1 < ntiles) step(k + 1, rb, ra);
    }
}

// ---------------- adjoint pass ----------------------------------------------
template <int NW>
struct BwdSmem {
    static constexpr int N = 16 * NW;
    alignas(16) float Bs[kT2][N];
    alignas(16) float Cs[kT2][N];
    float Dl[kT2], Aa[kT2], Dv[kT2];
    float xs[kT2][kP], dys[kT2][kP], xws[kT2][kP], zs[kT2][kP], dos[kT2][kP];
    float ycp[NW][kT2][kP], dxp[NW][kT2][kP], s1p[NW][kT2][kP];
    float red[3][NW];
};

template <typename Tin, typename Tout, int NW, bool SP>
__global__ __launch_bounds__(64 * NW) void m2_bwd_kernel(M2BwdArgs a) {
    constexpr int N = 16 * NW;
    constexpr int kPer = TileRegs<NW>::kPer;
    __shared__ BwdSmem<NW> sm;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int64_t bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
    const float Ah = a.A[h], biash = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const bool has_z = a.z != nullptr;
    const int64_t ntiles = (a.L + kT2 - 1) / kT2;

    float lam[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) lam[i] = 0.0f;
    float accD = 0.0f, accA = 0.0f, accBias = 0.0f;

    TileRegs<NW> nx;
    float4 ckn[4];
    auto load_ck = [&](int64_t k) {
        const float4* src =
            reinterpret_cast<const float4*>(a.ck + ((bh * ntiles + k) * NW + w) * (kP * 16)) + lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) ckn[q] = src[64 * q];
    };
    load_tile<Tin, Tout, NW, true>(a, b, h, g, (ntiles - 1) * kT2, nx);

    for (int64_t k = ntiles - 1; k >= 0; --k) {
        const int64_t t0 = k * kT2;
        // the tile's checkpoint, requested before the LDS staging below
        load_ck(k);
        // the tile's inputs, loaded during the tile after it, into LDS: B, C
        // rows, token constants, and per (token, channel) x, dout, z,
        // dy = dout silu(z) (or dout) and Delta x
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            (&sm.Bs[0][0])[tid + q * 64 * NW] = nx.b[q];
            (&sm.Cs[0][0])[tid + q * 64 * NW] = nx.c[q];
        }
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int j = w + m * NW;
            if (j < kT2) {
                float dl, av, dv;
                tok_consts<SP>(nx.dt[m], t0 + j < a.L, Ah, biash, dl, av, dv);
                if (lane == 0) {
                    sm.Dl[j] = dl;
                    sm.Aa[j] = av;
                    sm.Dv[j] = dv;
                }
                const float zz = nx.z[m];
                sm.xs[j][lane] = nx.x[m];
                sm.dos[j][lane] = nx.dout[m];
                sm.zs[j][lane] = zz;
                sm.dys[j][lane] = has_z ? nx.dout[m] * silu_scaled(zz, 1.0f) : nx.dout[m];
                sm.xws[j][lane] = dl * nx.x[m];
            }
        }
        float hc[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            hc[4 * q] = ckn[q].x; hc[4 * q + 1] = ckn[q].y; hc[4 * q + 2] = ckn[q].z; hc[4 * q + 3] = ckn[q].w;
        }
        lds_barrier();
        // the next tile's loads stay in flight over this tile's arithmetic
        if (k > 0) load_tile<Tin, Tout, NW, true>(a, b, h, g, (k - 1) * kT2, nx);

        // this wave's states at the tile's tokens, from its checkpoint
        float hs[kT2][16];
#pragma unroll
        for (int j = 0; j < kT2; ++j) {
            const float xw = sm.xws[j][lane], av = sm.Aa[j];
            const float4* br = reinterpret_cast<const float4*>(&sm.Bs[j][16 * w]);
            const float4* cr = reinterpret_cast<const float4*>(&sm.Cs[j][16 * w]);
            float yc = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 bb = br[q], cc = cr[q];
                const float bq[4] = {bb.x, bb.y, bb.z, bb.w}, cq[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * q + r;
                    hs[j][i] = __builtin_fmaf(av, j ? hs[j - 1][i] : hc[i], xw * bq[r]);
                    yc = __builtin_fmaf(cq[r], hs[j][i], yc);
                }
            }
            sm.ycp[w][j][lane] = yc;
        }

        // the adjoint back through the tile
#pragma unroll
        for (int j = kT2 - 1; j >= 0; --j) {
            const int64_t t = t0 + j;
            const float dy = sm.dys[j][lane], xw = sm.xws[j][lane], av = sm.Aa[j];
            const float4* br = reinterpret_cast<const float4*>(&sm.Bs[j][16 * w]);
            const float4* cr = reinterpret_cast<const float4*>(&sm.Cs[j][16 * w]);
            float vB[16], vC[16];
            float dxs = 0.0f, s1 = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 bb = br[q], cc = cr[q];
                const float bq[4] = {bb.x, bb.y, bb.z, bb.w}, cq[4] = {cc.x, cc.y, cc.z, cc.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * q + r;
                    const float l = __builtin_fmaf(dy, cq[r], lam[i]);
                    const float hp = j ? hs[j - 1][i] : hc[i];
                    vC[i] = dy * hs[j][i];
                    vB[i] = l * xw;
                    dxs = __builtin_fmaf(l, bq[r], dxs);
                    s1 = __builtin_fmaf(l, hp, s1);
                    lam[i] = av * l;
                }
            }
            sm.dxp[w][j][lane] = dxs;
            sm.s1p[w][j][lane] = s1;
            const float sBC = reduce32(vB, vC);
            if ((lane & 1) == 0 && t < a.L) {
                const int r = lane >> 4;   // rows 0, 1: dB; rows 2, 3: dC
                const int64_t o = (bh * a.L + t) * N + 16 * w + 8 * (r & 1) + ((lane >> 1) & 7);
                (r < 2 ? a.pB : a.pC)[o] = sBC;
            }
        }
        lds_barrier();

        // per (token, channel): dx, dz, and the token's dDelta (a wave per token)
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int j = w + m * NW;
            if (j >= kT2) continue;   // uniform per wave
            const int64_t t = t0 + j;
            const bool ok = t < a.L;
            float dxsum = 0.0f, s1sum = 0.0f, ycs = 0.0f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                dxsum += sm.dxp[v][j][lane];
                s1sum += sm.s1p[v][j][lane];
                ycs += sm.ycp[v][j][lane];
            }
            const float xv = sm.xs[j][lane], dy = sm.dys[j][lane];
            const float dl = sm.Dl[j], av = sm.Aa[j];
            const int64_t e = ((b * a.L + t) * a.H + h) * kP + lane;
            if (ok) a.dx[e] = __builtin_fmaf(dl, dxsum, Dh * dy);
            if (has_z && ok) {
                const float zz = sm.zs[j][lane];
                const float sg = fast_rcp(1.0f + fast_exp2(-zz * kLog2e));
                const float yc = __builtin_fmaf(Dh, xv, ycs);
                a.dz[e] = sm.dos[j][lane] * yc * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f);
            }
            accD = __builtin_fmaf(dy, xv, accD);
            accA = __builtin_fmaf(dl * av, s1sum, accA);
            const float ddl = wave_sum(__builtin_fmaf(xv, dxsum, Ah * av * s1sum));
            if (lane == 0 && ok) {
                const float dv = ddl * sm.Dv[j];
                a.ddt[(b * a.L + t) * a.H + h] = dv;
                accBias += dv;
            }
        }
        lds_barrier();   // the tile's LDS is rewritten next
    }

    if (a.dh0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) a.dh0[(bh * kP + lane) * N + 16 * w + i] = lam[i];
    }
    // the workgroup's shares of dD, dA, dbias
    accD = wave_sum(accD);
    accA = wave_sum(accA);
    if (lane == 0) {
        sm.red[0][w] = accD;
        sm.red[1][w] = accA;
        sm.red[2][w] = accBias;
    }
    lds_barrier();
    if (tid < 3) {
        float s = 0.0f;
        for (int v = 0; v < NW; ++v) s += sm.red[tid][v];
        (tid == 0 ? a.pD : tid == 1 ? a.pA : a.pbias)[bh] = s;
    }
}

// ---------------- chunked matrix form ---------------------------------------
// The same gradients regrouped over 32-token chunks as matrix products (the
// state-space-duality form the README's Mamba-2 section names), on the
// matrix cores.  With, inside a chunk, cum_t = A sum_{s <= t} Delta_s,
// F[t,s] = exp(cum_t - cum_s) Delta_s (s <= t, else 0), G = C B^T,
// M = G o F, W_s = exp(cum_last - cum_s) Delta_s, S_in the state entering
// the chunk (a checkpoint) and dS the adjoint of the state leaving it:
//   y       = M X + exp(cum) o (C S_in^T) + D X
//   dX      = M^T dY + W o (B dS^T) + D dY
//   dC      = (dM o F) B + (exp(cum) o dY) S_in,      dM = dY X^T
//   dB      = (dM o F)^T C + W o (X dS)
//   dS_in   = exp(cum_last) dS + (exp(cum) o dY)^T C
// and the scalar paths through F, exp(cum) and W collect into dcum_t and
// the direct dDelta_s; dDelta_s += A sum_{t >= s} dcum_t.  Every product is
// a v_mfma_f32_16x16x32_bf16 contraction.  Operands sit in LDS as bf16
// planes, row-major: x, B and C (bf16 inputs) exactly, the fp32 ones (dY,
// exp(cum) o dY, S_in, dS, M, dM o F) as hi + lo planes (hi*hi + hi*lo +
// lo*hi, relative error near 2^-16).  A fragment whose k runs along a row
// is one 16-byte read; one whose k runs down a column comes from two
// transposing reads (ds_read_b64_tr_b16).  bf16 inputs only.
constexpr int kQs = 32;    // tokens per chunk (4 checkpoint tiles)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_t;

__device__ __forceinline__ uint16_t bfbits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
__device__ __forceinline__ float bfval(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// v as a bf16 pair hi + lo
__device__ __forceinline__ void put2(uint16_t* hi, uint16_t* lo, float v) {
    const uint16_t hb = bfbits(v);
    *hi = hb;
    *lo = bfbits(v - bfval(hb));
}

// fragment of 8 consecutive k from a row (16-byte aligned)
__device__ __forceinline__ bf16x8_t frag_row(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}
// lane (g, i) of the wave: k = r0 + 8 g .. + 7 down column c0 + i of a
// row-major plane with row stride rs (two transposing reads)
__device__ __forceinline__ bf16x8_t frag_col(const uint16_t* m, int rs, int r0, int c0) {
    const int lane = threadIdx.x & 63, g = lane >> 4, a = lane & 15;
    const uint16_t* p = m + (r0 + 8 * g + (a >> 2)) * rs + c0 + 4 * (a & 3);
    const s16x4_t u = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(p));
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(p + 4 * rs));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(u, v, 0, 1, 2, 3, 4, 5, 6, 7));
}

// An MFMA operand in LDS: hi (and lo) planes, row stride rs; kc: k runs
// along the plane's rows (A: plane[row][k], B: plane[col][k]), else down
// its columns (A: plane[k][row], B: plane[k][col]).
struct Op {
    const uint16_t* hi;
    const uint16_t* lo;   // nullptr: exact in bf16
    int rs;
    bool kc;
};
__device__ __forceinline__ bf16x8_t frag(const Op& o, const uint16_t* plane, int idx0, int k0) {
    const int lane = threadIdx.x & 63;
    return o.kc ? frag_row(plane + (idx0 + (lane & 15)) * o.rs + k0 + 8 * (lane >> 4)) : frag_col(plane, o.rs, k0, idx0);
}
// acc += A[16 rows from r0] x B[16 cols from c0] over k = k0 .. k0 + K - 1
template <int K>
__device__ __forceinline__ f32x4_t mma(f32x4_t acc, const Op& A, int r0, const Op& B, int c0, int ka = 0, int kb = 0) {
#pragma unroll
    for (int kk = 0; kk < K; kk += 32) {
        const bf16x8_t ah = frag(A, A.hi, r0, ka + kk), bh = frag(B, B.hi, c0, kb + kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        if (B.lo) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, frag(B, B.lo, c0, kb + kk), acc, 0, 0, 0);
        if (A.lo) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag(A, A.lo, r0, ka + kk), bh, acc, 0, 0, 0);
    }
    return acc;
}

constexpr int kSsdThreads = 512;   // 8 waves: two per SIMD

template <int N>
struct SsdSmem {
    static constexpr int RP = kP + 8, RN = N + 16, RQ = kQs + 8;   // padded row strides (elements)
    alignas(16) uint16_t Xh[kQs][RP];
    alignas(16) uint16_t DYh[kQs][RP], DYl[kQs][RP];
    alignas(16) uint16_t EYh[kQs][RP], EYl[kQs][RP];       // exp(cum) o dY
    alignas(16) uint16_t Bh[kQs][RN], Ch[kQs][RN];
    alignas(16) uint16_t S0h[N][RP], S0l[N][RP];            // transposed: S_in^T[n][p]
    alignas(16) uint16_t dSh[N][RP], dSl[N][RP];            // transposed: dS^T[n][p]
    alignas(16) uint16_t Mh[kQs][RQ], Ml[kQs][RQ];
    alignas(16) uint16_t Kh[kQs][RQ], Kl[kQs][RQ];         // dM o F
    float Gm[kQs][kQs + 1], dM[kQs][kQs + 1];
    // token constants, double-buffered by chunk parity
    float dl[2][kQs], cum[2][kQs], em[2][kQs], dv[2][kQs];
    alignas(16) float ecum[2][kQs];
    alignas(16) float Wv[2][kQs];
    float Zf[kQs][kP];   // dout sigma(z) (1 + z (1 - sigma(z))): dz = Zf o (gate's input)
    float colp[kSsdThreads / 64][kQs], rowMM[kQs];   // per-wave column sums of V; row sums
    float dWp[N / 16][kQs], yyp[kP / 16][kQs];
    float red[8];
};

template <typename Tout, int N, bool SP>
__global__ __launch_bounds__(kSsdThreads) void m2_bwd_ssd_kernel(M2BwdArgs a) {
    constexpr int NW = N / 16, RP = SsdSmem<N>::RP, RN = SsdSmem<N>::RN, RQ = SsdSmem<N>::RQ;
    constexpr int TND = N / 16;                     // column tiles of the 64 x N state
    constexpr int NT = kSsdThreads, NWV = NT / 64;   // threads, waves
    constexpr int TPW = 4 * TND / NWV;              // state tiles per wave
    __shared__ SsdSmem<N> sm;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, gq = lane >> 4, li = lane & 15;
    const int64_t bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
    const float Ah = a.A[h], biash = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float Dh = a.D ? a.D[h] : 0.0f;
    const bool has_z = a.z != nullptr;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* Zp = reinterpret_cast<const uint16_t*>(a.z);
    const uint16_t* DT = reinterpret_cast<const uint16_t*>(a.dt);
    const uint16_t* Bp = reinterpret_cast<const uint16_t*>(a.B);
    const uint16_t* Cp = reinterpret_cast<const uint16_t*>(a.C);
    const Tout* DO = reinterpret_cast<const Tout*>(a.dout);
    const int64_t nch = (a.L + kQs - 1) / kQs;

    const Op opX{&sm.Xh[0][0], nullptr, RP, true}, opXt{&sm.Xh[0][0], nullptr, RP, false};
    const Op opDYt{&sm.DYh[0][0], &sm.DYl[0][0], RP, false}, opDY{&sm.DYh[0][0], &sm.DYl[0][0], RP, true};
    const Op opEY{&sm.EYh[0][0], &sm.EYl[0][0], RP, true}, opEYt{&sm.EYh[0][0], &sm.EYl[0][0], RP, false};
    const Op opB{&sm.Bh[0][0], nullptr, RN, true}, opBt{&sm.Bh[0][0], nullptr, RN, false};
    const Op opC{&sm.Ch[0][0], nullptr, RN, true}, opCt{&sm.Ch[0][0], nullptr, RN, false};
    const Op opS0{&sm.S0h[0][0], &sm.S0l[0][0], RP, false}, opS0t{&sm.S0h[0][0], &sm.S0l[0][0], RP, true};
    const Op opdS{&sm.dSh[0][0], &sm.dSl[0][0], RP, false}, opdSt{&sm.dSh[0][0], &sm.dSl[0][0], RP, true};
    const Op opM{&sm.Mh[0][0], &sm.Ml[0][0], RQ, true}, opMt{&sm.Mh[0][0], &sm.Ml[0][0], RQ, false};
    const Op opK{&sm.Kh[0][0], &sm.Kl[0][0], RQ, true}, opKt{&sm.Kh[0][0], &sm.Kl[0][0], RQ, false};

    // the adjoint of the state leaving the current chunk: this wave's tiles
    // (tile wv + NWV j of the 4 x TND tiles of 16 x 16) in registers
    f32x4_t dSr[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) dSr[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int e = tid; e < N * RP; e += NT) {
        (&sm.dSh[0][0])[e] = 0;
        (&sm.dSl[0][0])[e] = 0;
    }
    float accD = 0.0f, accA = 0.0f, accBias = 0.0f;

    // a chunk's global inputs as 16-byte loads into registers, fetched while
    // the chunk after it (the one before in this reverse walk) is computed
    constexpr int SEG = N / 8, NBC = (kQs * SEG + NT - 1) / NT;
    const int st = tid >> 4, sq = tid & 15;   // token, 4-channel segment
    uint2 xr, zr;
    uint4 br[NBC], cr[NBC];
    float dov[4];
    uint32_t dtr;   // dt's bf16 bits
    float4 ckr[NW / 2];
    auto fetch = [&](int64_t c) {
        const int64_t t0 = c * kQs;
        const bool sok = t0 + st < a.L;
        const int64_t sgi = ((b * a.L + t0 + st) * a.H + h) * kP + 4 * sq;
        xr = zr = uint2{0u, 0u};
        if constexpr (sizeof(Tout) == 4) {
            float4 d0 = {0.0f, 0.0f, 0.0f, 0.0f};
            if (sok) d0 = *reinterpret_cast<const float4*>(DO + sgi);
            dov[0] = d0.x; dov[1] = d0.y; dov[2] = d0.z; dov[3] = d0.w;
        } else {
            uint2 dr = {0u, 0u};
            if (sok) dr = *reinterpret_cast<const uint2*>(DO + sgi);
            const uint32_t w2[2] = {dr.x, dr.y};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                dov[2 * i] = __uint_as_float(w2[i] << 16);
                dov[2 * i + 1] = __uint_as_float(w2[i] & 0xffff0000u);
            }
        }
        if (sok) {
            xr = *reinterpret_cast<const uint2*>(X + sgi);
            if (has_z) zr = *reinterpret_cast<const uint2*>(Zp + sgi);
        }
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            const int e = tid + NT * i, t = e / SEG, sg8 = e - t * SEG;
            br[i] = cr[i] = uint4{0u, 0u, 0u, 0u};
            if (e < kQs * SEG && t0 + t < a.L) {
                const int64_t gi = ((b * a.L + t0 + t) * a.G + g) * N + 8 * sg8;
                br[i] = *reinterpret_cast<const uint4*>(Bp + gi);
                cr[i] = *reinterpret_cast<const uint4*>(Cp + gi);
            }
        }
        const float4* src = reinterpret_cast<const float4*>(a.ck + (bh * nch + c) * (int64_t)(NW * kP * 16));
#pragma unroll
        for (int i = 0; i < NW / 2; ++i) ckr[i] = src[NT * i + tid];
        // raw bits: converting here would make the wave wait for the load at once
        dtr = 0u;
        if (wv == 1 && lane < kQs && t0 + lane < a.L) dtr = DT[(b * a.L + t0 + lane) * a.H + h];
    };
    fetch(nch - 1);

    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t t0 = c * kQs;
        const int tb = (int)(c & 1);   // this chunk's token constants
        // ---- stage: x, B, C (exact), dY and S_in to their planes, dout's
        //      gate factor to Zf, from the registers fetched during the chunk after
        *reinterpret_cast<uint2*>(&sm.Xh[st][4 * sq]) = xr;
        {
            const uint32_t zw[2] = {zr.x, zr.y};
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                uint32_t hp = 0u, lp = 0u;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int j = 2 * i + k;
                    float dy = dov[j];
                    if (has_z) {
                        const float zz = __uint_as_float(k ? (zw[i] & 0xffff0000u) : (zw[i] << 16));
                        const float sg = fast_rcp(1.0f + fast_exp2(-zz * kLog2e));
                        sm.Zf[st][4 * sq + j] = dov[j] * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f);
                        dy = dov[j] * zz * sg;
                    }
                    const uint16_t hb = bfbits(dy), lb = bfbits(dy - bfval(hb));
                    hp |= (uint32_t)hb << (16 * k);
                    lp |= (uint32_t)lb << (16 * k);
                }
                hw[i] = hp;
                lw[i] = lp;
            }
            *reinterpret_cast<uint2*>(&sm.DYh[st][4 * sq]) = uint2{hw[0], hw[1]};
            *reinterpret_cast<uint2*>(&sm.DYl[st][4 * sq]) = uint2{lw[0], lw[1]};
        }
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            const int e = tid + NT * i, t = e / SEG, sg8 = e - t * SEG;
            if (e < kQs * SEG) {
                *reinterpret_cast<uint4*>(&sm.Bh[t][8 * sg8]) = br[i];
                *reinterpret_cast<uint4*>(&sm.Ch[t][8 * sg8]) = cr[i];
            }
        }
#pragma unroll
        for (int i = 0; i < NW / 2; ++i) {
            // record float4 (n block, p block, q, i): rows p = 16 p block + 4 q .. + 3
            // of the state's column n = 16 n block + i
            const int e4 = NT * i + tid, n = 16 * (e4 >> 8) + (e4 & 15), p = 16 * ((e4 >> 6) & 3) + 4 * ((e4 >> 4) & 3);
            const float v[4] = {ckr[i].x, ckr[i].y, ckr[i].z, ckr[i].w};
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint16_t h0b = bfbits(v[2 * i]), h1b = bfbits(v[2 * i + 1]);
                hw[i] = (uint32_t)h0b | ((uint32_t)h1b << 16);
                lw[i] = (uint32_t)bfbits(v[2 * i] - bfval(h0b)) | ((uint32_t)bfbits(v[2 * i + 1] - bfval(h1b)) << 16);
            }
            *reinterpret_cast<uint2*>(&sm.S0h[n][p]) = uint2{hw[0], hw[1]};
            *reinterpret_cast<uint2*>(&sm.S0l[n][p]) = uint2{lw[0], lw[1]};
        }
        if (wv == 1 && lane < kQs) {   // wave 0 may still be on the chunk after's scalars
            float dl, av, dvv;
            const bool ok = t0 + lane < a.L;
            tok_consts<SP>(__uint_as_float(dtr << 16), ok, Ah, biash, dl, av, dvv);
            float cs = dl * Ah;   // inclusive prefix of Delta A over the chunk
#pragma unroll
            for (int o = 1; o < kQs; o <<= 1) {
                const float up = __shfl_up(cs, o, 64);
                if (lane >= o) cs += up;
            }
            const float cl = __shfl(cs, kQs - 1, 64);
            sm.dl[tb][lane] = dl;
            sm.cum[tb][lane] = cs;
            sm.ecum[tb][lane] = __expf(cs);
            sm.em[tb][lane] = __expf(cl - cs);
            sm.Wv[tb][lane] = __expf(cl - cs) * dl;
            sm.dv[tb][lane] = dvv;
        }
        if (c > 0) fetch(c - 1);
        lds_barrier();

        auto F = [&](int t, int s) { return s <= t ? __expf(sm.cum[tb][t] - sm.cum[tb][s]) * sm.dl[tb][s] : 0.0f; };
        // ---- G = C B^T, M = G o F (tiles 0..3); dM = dY X^T (tiles 4..7); exp(cum) o dY
        for (int tile = wv; tile < 8; tile += NWV) {
            const int tm = (tile >> 1) & 1, tn = tile & 1;
            f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
            if (tile < 4) {
                acc = mma<N>(acc, opC, 16 * tm, opB, 16 * tn);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tm + 4 * gq + r, s = 16 * tn + li;
                    sm.Gm[t][s] = acc[r];
                    put2(&sm.Mh[t][s], &sm.Ml[t][s], acc[r] * F(t, s));
                }
            } else {
                acc = mma<kP>(acc, opDY, 16 * tm, opX, 16 * tn);
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.dM[16 * tm + 4 * gq + r][16 * tn + li] = acc[r];
            }
        }
        for (int e = tid; e < kQs * kP / 4; e += NT) {   // 4 channels of one token per thread
            const int t = e >> 4, p = 4 * (e & 15);
            const uint2 hv = *reinterpret_cast<const uint2*>(&sm.DYh[t][p]);
            const uint2 lv = *reinterpret_cast<const uint2*>(&sm.DYl[t][p]);
            const float ec = sm.ecum[tb][t];
            const uint32_t hw[2] = {hv.x, hv.y}, lw[2] = {lv.x, lv.y};
            uint32_t oh[2], ol[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float v0 = ec * (__uint_as_float(hw[i] << 16) + __uint_as_float(lw[i] << 16));
                const float v1 = ec * (__uint_as_float(hw[i] & 0xffff0000u) + __uint_as_float(lw[i] & 0xffff0000u));
                const uint16_t h0b = bfbits(v0), h1b = bfbits(v1);
                oh[i] = (uint32_t)h0b | ((uint32_t)h1b << 16);
                ol[i] = (uint32_t)bfbits(v0 - bfval(h0b)) | ((uint32_t)bfbits(v1 - bfval(h1b)) << 16);
            }
            *reinterpret_cast<uint2*>(&sm.EYh[t][p]) = uint2{oh[0], oh[1]};
            *reinterpret_cast<uint2*>(&sm.EYl[t][p]) = uint2{ol[0], ol[1]};
        }
        lds_barrier();

        // ---- y (for dz) = M X + exp(cum) o (C S_in^T) + D x, with its dY . Yint row sums;
        //      dX = M^T dY + W o (B dS^T) + D dY;   dM o F;   scalar sums
        for (int tile = wv; tile < 8; tile += NWV) {
            const int tm = tile >> 2, tn = tile & 3;
            f32x4_t yi = mma<kQs>(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, opM, 16 * tm, opXt, 16 * tn);
            f32x4_t y0 = mma<N>(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, opC, 16 * tm, opS0, 16 * tn);
            f32x4_t d1 = mma<kQs>(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, opMt, 16 * tm, opDYt, 16 * tn);
            f32x4_t d2 = mma<N>(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, opB, 16 * tm, opdS, 16 * tn);
            const float4 ec4 = *reinterpret_cast<const float4*>(&sm.ecum[tb][16 * tm + 4 * gq]);
            const float4 wv4 = *reinterpret_cast<const float4*>(&sm.Wv[tb][16 * tm + 4 * gq]);
            const float ecr[4] = {ec4.x, ec4.y, ec4.z, ec4.w}, wvr[4] = {wv4.x, wv4.y, wv4.z, wv4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tm + 4 * gq + r, p = 16 * tn + li;
                const bool ok = t0 + t < a.L;
                const int64_t gi = ((b * a.L + t0 + t) * a.H + h) * kP + p;
                const float xv = bfval(sm.Xh[t][p]), dy = bfval(sm.DYh[t][p]) + bfval(sm.DYl[t][p]);
                const float yint = ecr[r] * y0[r];
                if (has_z && ok) a.dz[gi] = sm.Zf[t][p] * (yi[r] + yint + Dh * xv);
                if (ok) accD = __builtin_fmaf(dy, xv, accD);
                if (ok) a.dx[gi] = d1[r] + wvr[r] * d2[r] + Dh * dy;
                const float yy = row_sum(dy * yint);
                if (li == 0) sm.yyp[tn][t] = yy;
            }
        }
        // dM o F into its planes, and the sums over V = dM o G o exp(cum_t - cum_s)
        // below the diagonal (s < t): rowMM_t = sum_s V Delta_s here, the column
        // sums sum_t V as one partial per wave.  The diagonal enters dcum_t
        // twice with opposite signs and is left out of both; the direct
        // dDelta_s adds it back.  Thread: token t, columns 2 sb, 2 sb + 1.
        {
            const int t = tid >> 4, sb = tid & 15;
            const float ct = sm.cum[tb][t];
            float vs[2], row = 0.0f;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int s = 2 * sb + k;
                const float e = s <= t ? __expf(ct - sm.cum[tb][s]) : 0.0f;
                const float dm = sm.dM[t][s];
                put2(&sm.Kh[t][s], &sm.Kl[t][s], dm * e * sm.dl[tb][s]);
                vs[k] = s < t ? dm * sm.Gm[t][s] * e : 0.0f;
                row = __builtin_fmaf(vs[k], sm.dl[tb][s], row);
            }
            row += __shfl_xor(row, 1, 64);
            row += __shfl_xor(row, 2, 64);
            row += __shfl_xor(row, 4, 64);
            row += __shfl_xor(row, 8, 64);
            if (sb == 0) sm.rowMM[t] = row;
#pragma unroll
            for (int k = 0; k < 2; ++k) {   // over the wave's 4 tokens
                vs[k] += __shfl_xor(vs[k], 16, 64);
                vs[k] += __shfl_xor(vs[k], 32, 64);
            }
            if (lane < 16) {
#pragma unroll
                for (int k = 0; k < 2; ++k) sm.colp[wv][2 * lane + k] = vs[k];
            }
        }
        lds_barrier();

        // ---- dC = (dM o F) B + (exp(cum) o dY) S_in;  dB = (dM o F)^T C + W o (X dS), dW
        for (int tile = wv; tile < 2 * TND; tile += NWV) {
            const int tm = tile / TND, tn = tile - tm * TND;
            f32x4_t dc = mma<kQs>(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, opK, 16 * tm, opBt, 16 * tn);
            dc = mma<kP>(dc, opEY, 16 * tm, opS0t, 16 * tn);
            const f32x4_t db = mma<kQs>(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, opKt, 16 * tm, opCt, 16 * tn);
            const f32x4_t xd = mma<kP>(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, opX, 16 * tm, opdSt, 16 * tn);
            const float4 wv4 = *reinterpret_cast<const float4*>(&sm.Wv[tb][16 * tm + 4 * gq]);
            const float wvr[4] = {wv4.x, wv4.y, wv4.z, wv4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * tm + 4 * gq + r, n = 16 * tn + li;
                if (t0 + s < a.L) {
                    a.pC[(bh * a.L + t0 + s) * N + n] = dc[r];
                    a.pB[(bh * a.L + t0 + s) * N + n] = db[r] + wvr[r] * xd[r];
                }
                const float part = row_sum(xd[r] * bfval(sm.Bh[s][n]));
                if (li == 0) sm.dWp[tn][s] = part;
            }
        }
        // sum_{p,n} dS o S_in (the exp(cum_last) path), this wave's tiles
        float sds = 0.0f;
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wv + NWV * j, tm = tile / TND, tn = tile - tm * TND;
            const int p = 16 * tm + 4 * gq, n = 16 * tn + li;   // rows p .. p + 3 of column n
            const uint2 h2 = *reinterpret_cast<const uint2*>(&sm.S0h[n][p]);
            const uint2 l2 = *reinterpret_cast<const uint2*>(&sm.S0l[n][p]);
            const uint32_t hw[2] = {h2.x, h2.y}, lw[2] = {l2.x, l2.y};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t hb = (r & 1) ? (hw[r >> 1] & 0xffff0000u) : (hw[r >> 1] << 16);
                const uint32_t lb = (r & 1) ? (lw[r >> 1] & 0xffff0000u) : (lw[r >> 1] << 16);
                sds += dSr[j][r] * (__uint_as_float(hb) + __uint_as_float(lb));
            }
        }
        sds = wave_sum(sds);
        if (lane == 0) sm.red[wv] = sds;
        lds_barrier();

        // ---- dS_in = exp(cum_last) dS + (exp(cum) o dY)^T C, into registers and the planes
        {
            const float ecl = sm.ecum[tb][kQs - 1];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int tile = wv + NWV * j, tm = tile / TND, tn = tile - tm * TND;
                const f32x4_t u = mma<kQs>(f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, opEYt, 16 * tm, opCt, 16 * tn);
                uint16_t hb[4], lb[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dSr[j][r] = __builtin_fmaf(ecl, dSr[j][r], u[r]);
                    hb[r] = bfbits(dSr[j][r]);
                    lb[r] = bfbits(dSr[j][r] - bfval(hb[r]));
                }
                // rows p = 16 tm + 4 gq .. + 3 of column n: four consecutive p of dS^T
                const int p = 16 * tm + 4 * gq, n = 16 * tn + li;
                *reinterpret_cast<uint2*>(&sm.dSh[n][p]) =
                    uint2{(uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16)};
                *reinterpret_cast<uint2*>(&sm.dSl[n][p]) =
                    uint2{(uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16)};
            }
        }
        lds_barrier();
        // ---- per token: dcum, dDelta, ddt, and the chunk's share of dA, dbias, dD
        //      (wave 0, while the others stage the next chunk: nothing it reads
        //      is written before the next chunk's first barrier)
        if (wv == 0) {
            const int t = lane;
            float dW = 0.0f, dc = 0.0f, dDl = 0.0f;
            if (t < kQs) {
                float yy = 0.0f;
                for (int tn = 0; tn < kP / 16; ++tn) yy += sm.yyp[tn][t];
                for (int tn = 0; tn < N / 16; ++tn) dW += sm.dWp[tn][t];
                float col = 0.0f;
#pragma unroll
                for (int w = 0; w < NWV; ++w) col += sm.colp[w][t];
                dDl = col + sm.dM[t][t] * sm.Gm[t][t];
                dc = sm.rowMM[t] - sm.dl[tb][t] * col + yy - dW * sm.Wv[tb][t];
            }
            // the last token also carries exp(cum_last)'s paths: sum_s dW_s W_s
            // and exp(cum_last) sum dS o S_in
            const float dwW = wave_sum(t < kQs ? dW * sm.Wv[tb][t] : 0.0f);
            float sds_all = 0.0f;
#pragma unroll
            for (int w = 0; w < NWV; ++w) sds_all += sm.red[w];
            if (t == kQs - 1) dc += dwW + sm.ecum[tb][kQs - 1] * sds_all;
            // rc_t = sum_{t' >= t} dcum_t' (a reversed inclusive scan over the lanes)
            float rc = t < kQs ? dc : 0.0f;
#pragma unroll
            for (int o = 1; o < kQs; o <<= 1) {
                const float dn = __shfl_down(rc, o, 64);
                if (t + o < kQs) rc += dn;
            }
            if (t < kQs && t0 + t < a.L) {
                const float dD = dDl + dW * sm.em[tb][t] + Ah * rc;
                const float dvt = dD * sm.dv[tb][t];
                a.ddt[(b * a.L + t0 + t) * a.H + h] = dvt;
                accBias += dvt;
                accA = __builtin_fmaf(sm.dl[tb][t], rc, accA);
            }
        }
    }
    lds_barrier();   // wave 0 reads red above
    if (a.dh0) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int tile = wv + NWV * j, tm = tile / TND, tn = tile - tm * TND;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.dh0[(bh * kP + 16 * tm + 4 * gq + r) * N + 16 * tn + li] = dSr[j][r];
        }
    }
    // dD = sum dY o x: every wave holds a share
    accD = wave_sum(accD);
    if (lane == 0) sm.red[wv] = accD;
    lds_barrier();
    if (wv == 0) {
        accD = 0.0f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) accD += sm.red[w];
        accA = wave_sum(accA);
        accBias = wave_sum(accBias);
        if (lane == 0) {
            a.pD[bh] = accD;
            a.pA[bh] = accA;
            a.pbias[bh] = accBias;
        }
    }
}

// ---------------- chunk-entry states on the matrix cores --------------------
// The chunked form needs only the state entering each chunk, and each
// follows from the one before by a single product:
//   S_out = exp(cum_last) S_in + (W o X)^T B,   W_s = exp(cum_last - cum_s) Delta_s.
// The state S[p][n] is held as MFMA accumulators (rows p, columns n): a
// lane's four rows are four consecutive p of one n, which is one float4 of
// the record and, transposed, one 8-byte row piece of the consumer's
// S_in^T planes.  Eight waves (two per SIMD): wave w owns the rows
// p = 16 (w & 3) .. + 15 and half of the columns n.  The next chunk's
// inputs are loaded while this one is multiplied, and the LDS operands are
// double-buffered so that one chunk's writes never meet the other's reads.
template <int N, bool SP>
__global__ __launch_bounds__(512) void m2_bwd_chunk_state_kernel(M2BwdArgs a) {
    constexpr int NW = N / 16, SEG = N / 8, NT = 512, NBC = (kQs * SEG + NT - 1) / NT, NJ = NW / 2;
    constexpr int RP = kP + 8, RN = N + 16;
    __shared__ alignas(16) uint16_t Bh[2][kQs][RN];
    __shared__ alignas(16) uint16_t XWh[2][kQs][RP];
    __shared__ alignas(16) uint16_t XWl[2][kQs][RP];
    __shared__ float Ws[2][kQs], Es[2];
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, gq = lane >> 4, li = lane & 15;
    const int64_t bh = blockIdx.x, b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
    const float Ah = a.A[h], biash = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* Bp = reinterpret_cast<const uint16_t*>(a.B);
    const uint16_t* DT = reinterpret_cast<const uint16_t*>(a.dt);
    const int64_t nch = (a.L + kQs - 1) / kQs;
    const int st = tid >> 4, sq = tid & 15;   // token, 4-channel segment of x
    const int pb = wv & 3, j0 = (wv >> 2) * NJ;   // this wave's column block, first row block

    f32x4_t acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[j][r] = a.h0 ? a.h0[(bh * kP + 16 * pb + 4 * gq + r) * N + 16 * (j0 + j) + li] : 0.0f;

    uint2 xr;
    uint4 br[NBC];
    uint32_t dtr;   // dt's bf16 bits
    auto load = [&](int64_t c) {
        const int64_t t0 = c * kQs;
        xr = uint2{0u, 0u};
        if (t0 + st < a.L) xr = *reinterpret_cast<const uint2*>(X + ((b * a.L + t0 + st) * a.H + h) * kP + 4 * sq);
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            const int e = tid + NT * i, t = e / SEG, s8 = e - t * SEG;
            br[i] = uint4{0u, 0u, 0u, 0u};
            if (e < kQs * SEG && t0 + t < a.L)
                br[i] = *reinterpret_cast<const uint4*>(Bp + ((b * a.L + t0 + t) * a.G + g) * N + 8 * s8);
        }
        // raw bits: converting here would make the wave wait for the load at once
        dtr = 0u;
        if (wv == 0 && lane < kQs && t0 + lane < a.L) dtr = DT[(b * a.L + t0 + lane) * a.H + h];
    };
    if (nch > 1) load(0);
    for (int64_t c = 0; c < nch; ++c) {
        float4* dst = reinterpret_cast<float4*>(a.ck + (bh * nch + c) * (int64_t)(NW * kP * 16));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            dst[256 * (j0 + j) + 64 * pb + 16 * gq + li] = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
        if (c + 1 == nch) break;
        const int buf = (int)(c & 1);
        if (wv == 0 && lane < kQs) {
            float dl, av, dvv;
            tok_consts<SP>(__uint_as_float(dtr << 16), c * kQs + lane < a.L, Ah, biash, dl, av, dvv);
            float cs = dl * Ah;   // inclusive prefix of Delta A over the chunk
#pragma unroll
            for (int o = 1; o < kQs; o <<= 1) {
                const float up = __shfl_up(cs, o, 64);
                if (lane >= o) cs += up;
            }
            const float cl = __shfl(cs, kQs - 1, 64);
            Ws[buf][lane] = __expf(cl - cs) * dl;
            if (lane == 0) Es[buf] = __expf(cl);
        }
#pragma unroll
        for (int i = 0; i < NBC; ++i) {
            const int e = tid + NT * i, t = e / SEG, s8 = e - t * SEG;
            if (e < kQs * SEG) *reinterpret_cast<uint4*>(&Bh[buf][t][8 * s8]) = br[i];
        }
        const uint2 xc = xr;
        if (c + 2 < nch) load(c + 1);   // the last chunk never updates the state
        lds_barrier();
        {
            const float wt = Ws[buf][st];
            const uint32_t xw4[2] = {xc.x, xc.y};
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float v0 = wt * __uint_as_float(xw4[i] << 16), v1 = wt * __uint_as_float(xw4[i] & 0xffff0000u);
                const uint16_t h0b = bfbits(v0), h1b = bfbits(v1);
                hw[i] = (uint32_t)h0b | ((uint32_t)h1b << 16);
                lw[i] = (uint32_t)bfbits(v0 - bfval(h0b)) | ((uint32_t)bfbits(v1 - bfval(h1b)) << 16);
            }
            *reinterpret_cast<uint2*>(&XWh[buf][st][4 * sq]) = uint2{hw[0], hw[1]};
            *reinterpret_cast<uint2*>(&XWl[buf][st][4 * sq]) = uint2{lw[0], lw[1]};
        }
        lds_barrier();
        const float ecl = Es[buf];
        const bf16x8_t xh = frag_col(&XWh[buf][0][0], RP, 0, 16 * pb);
        const bf16x8_t xl = frag_col(&XWl[buf][0][0], RP, 0, 16 * pb);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const bf16x8_t bf = frag_col(&Bh[buf][0][0], RN, 0, 16 * (j0 + j));
            f32x4_t s = acc[j] * ecl;
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bf, s, 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bf, s, 0, 0, 0);
        }
    }
}

// dB, dC: sums of the per-head partials over the heads of each group, one
// thread per (batch, token, group, n).
__global__ __launch_bounds__(256) void m2_bwd_bc_reduce_kernel(M2BwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = a.batch * a.L * a.G * a.N;
    if (i >= total) return;
    const int64_t n = i % a.N, r = i / a.N, g = r % a.G, bt = r / a.G, t = bt % a.L, b = bt / a.L;
    const int64_t hpg = a.H / a.G;
    float sB = 0.0f, sC = 0.0f;
    for (int64_t hh = g * hpg; hh < (g + 1) * hpg; ++hh) {
        const int64_t o = ((b * a.H + hh) * a.L + t) * a.N + n;
        sB += a.pB[o];
        sC += a.pC[o];
    }
    a.dB[i] = sB;
    a.dC[i] = sC;
}

// dA, dD, dbias: sums over batches of the per-(batch, head) partials.
__global__ __launch_bounds__(64) void m2_bwd_param_reduce_kernel(M2BwdArgs a) {
    const int64_t h = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (h >= a.H) return;
    float sA = 0.0f, sD = 0.0f, sb = 0.0f;
    for (int64_t b = 0; b < a.batch; ++b) {
        sA += a.pA[b * a.H + h];
        sD += a.pD[b * a.H + h];
        sb += a.pbias[b * a.H + h];
    }
    a.dA[h] = sA;
    if (a.dD) a.dD[h] = a.D ? sD : 0.0f;
    if (a.ddt_bias) a.ddt_bias[h] = a.dt_bias ? sb : 0.0f;
}

template <typename Tin, typename Tout, int NW>
hipError_t launch_nw(M2BwdArgs a, bool ssd, hipStream_t stream) {
    const dim3 grid((unsigned)(a.batch * a.H)), block(64 * NW);
    // the chunked form takes bf16 inputs, N >= 32 and 16-byte aligned x, z, dout, B, C
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    ssd = ssd && NW >= 2 && sizeof(Tin) == 2 && al16(a.x) && al16(a.z) && al16(a.dout) && al16(a.B) && al16(a.C);
    if constexpr (NW >= 2 && sizeof(Tin) == 2) {
        if (ssd) {
            {
                KTime kt("m2_bwd_chunk_state", stream);
                if (a.softplus)
                    hipLaunchKernelGGL((m2_bwd_chunk_state_kernel<16 * NW, true>), grid, dim3(512), 0, stream, a);
                else
                    hipLaunchKernelGGL((m2_bwd_chunk_state_kernel<16 * NW, false>), grid, dim3(512), 0, stream, a);
            }
            KTime kt("m2_bwd_ssd", stream);
            if (a.softplus)
                hipLaunchKernelGGL((m2_bwd_ssd_kernel<Tout, 16 * NW, true>), grid, dim3(kSsdThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((m2_bwd_ssd_kernel<Tout, 16 * NW, false>), grid, dim3(kSsdThreads), 0, stream, a);
            return hipGetLastError();
        }
    }
    {
        KTime kt("m2_bwd_checkpoint", stream);
        if (a.softplus)
            hipLaunchKernelGGL((m2_bwd_ck_kernel<Tin, NW, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((m2_bwd_ck_kernel<Tin, NW, false>), grid, block, 0, stream, a);
    }
    {
        KTime kt("m2_bwd_adjoint", stream);
        if (a.softplus)
            hipLaunchKernelGGL((m2_bwd_kernel<Tin, Tout, NW, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((m2_bwd_kernel<Tin, Tout, NW, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_dt(const M2BwdArgs& a, bool ssd, hipStream_t stream) {
    switch (a.N) {
        case 16: return launch_nw<Tin, Tout, 1>(a, false, stream);
        case 32: return launch_nw<Tin, Tout, 2>(a, ssd, stream);
        case 64: return launch_nw<Tin, Tout, 4>(a, ssd, stream);
        default: return launch_nw<Tin, Tout, 8>(a, ssd, stream);
    }
}

}  // namespace

size_t m2_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t N) {
    const int64_t ntiles = (L + kT2 - 1) / kT2;
    const int64_t ck = batch * H * ntiles * kP * N;      // checkpoints
    const int64_t part = 2 * batch * H * L * N;          // per-head dB, dC
    const int64_t par = 3 * batch * H;                   // per-(batch, head) dD, dA, dbias
    return (size_t)(ck + part + par + 64) * sizeof(float);
}

void m2_bwd_carve(M2BwdArgs& a, void* ws) {
    float* p = static_cast<float*>(ws);
    const int64_t ntiles = (a.L + kT2 - 1) / kT2;
    a.ck = p;
    p += a.batch * a.H * ntiles * kP * a.N;
    a.pB = p;
    p += a.batch * a.H * a.L * a.N;
    a.pC = p;
    p += a.batch * a.H * a.L * a.N;
    a.pA = p;
    a.pD = p + a.batch * a.H;
    a.pbias = p + 2 * a.batch * a.H;
}

hipError_t launch_m2_bwd(const M2BwdArgs& a, int in_bf16, int out_bf16, int ssd, hipStream_t stream) {
    hipError_t e;
    if (in_bf16)
        e = out_bf16 ? launch_dt<uint16_t, uint16_t>(a, ssd, stream) : launch_dt<uint16_t, float>(a, ssd, stream);
    else
        e = out_bf16 ? launch_dt<float, uint16_t>(a, ssd, stream) : launch_dt<float, float>(a, ssd, stream);
    if (e != hipSuccess) return e;
    {
        KTime kt("m2_bwd_bc_reduce", stream);
        const int64_t total = a.batch * a.L * a.G * a.N;
        hipLaunchKernelGGL(m2_bwd_bc_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a);
    }
    {
        KTime kt("m2_bwd_param_reduce", stream);
        hipLaunchKernelGGL(m2_bwd_param_reduce_kernel, dim3((unsigned)((a.H + 63) / 64)), dim3(64), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace selscan
