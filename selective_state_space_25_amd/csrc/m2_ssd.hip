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
// Two kernels share this arithmetic:
//  - m2_ssd_ws_kernel (the default) splits the roles: four state waves hold
//    the state and compute C S, the gate and y, and the state update; four
//    chunk waves build M and M X and stage the inputs one chunk ahead, with
//    one barrier per chunk between the groups (see its comment);
//  - m2_ssd_kernel has every wave take part in every step, with four
//    barrier-separated phases per chunk.  Wave w holds the state rows of one
//    half of n (w / 4) for 16 columns (w % 4) in accumulator tiles, and
//    computes its part of C S (straight from those registers), of M X and of
//    the state update; two LDS buffers collect the two halves' parts of Y.
//    Every thread also stages an eighth of a token's inputs, builds M tiles,
//    splits the weighted x, prepares the gate and writes y.
// Chunk inputs stay in LDS in their memory layout ([token][channel] rows);
// operands that need the other orientation are read with the transposing LDS
// load (ds_read_b64_tr_b16), which hands each lane four consecutive rows of
// one column.  Global memory is read and written through buffer descriptors
// bounded at the last token, so tokens past L load as zero and their stores
// are dropped by the hardware: every chunk issues the same memory
// operations.
#include <type_traits>

#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4;

constexpr int kQ = 64;                     // tokens per chunk
constexpr int kPd = 64;                    // headdim handled by this kernel
constexpr int kWaves = 8;                  // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRowX = kPd + 8;             // padded row (elements) of x, z, weighted x
constexpr int kRowM = kQ + 8;              // padded row of M
constexpr int kRowY = kPd + 4;             // padded row (floats) of Y
constexpr int kBufWord3 = 0x00020000;      // buffer descriptor word 3: 32-bit data format, raw access

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

// A buffer descriptor over `rows` rows of `row_bytes` bytes spaced `stride`
// bytes apart from p: accesses at or past the last row's end read zero and
// drop their stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* p, int64_t rows, int64_t stride,
                                                           int row_bytes) {
    const int n = rows > 0 ? (int)((rows - 1) * stride + row_bytes) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, kBufWord3);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

// Eight consecutive k of an MFMA operand from two 4-element pieces.
__device__ __forceinline__ bf16x8 cat(s16x4 a, s16x4 b) {
    const s16x8 r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
}

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

// B and C rows sit in LDS with the state index permuted in 4-element
// pieces inside each group of 32: pieces 0..7 at positions 0, 2, 4, 6, 1, 3,
// 5, 7.  The C operand of C S takes pieces p and p + 4 of a group (the
// order that matches the state's accumulator rows), which are then one
// contiguous 16-byte read instead of two 8-byte reads from 16 rows (2-way
// bank conflicts); the contractions over n pair B and C under the same
// permutation, and the transposed B reads address their pieces through it.
__device__ __forceinline__ int npos(int n) {
    const int pc = (n & 31) >> 2;
    return (n & ~31) + 4 * (pc < 4 ? 2 * pc : 2 * pc - 7) + (n & 3);
}

// As ld_col8 over a B row block stored with npos: columns c0 .. c0 + 15.
__device__ __forceinline__ bf16x8 ld_col8_n(const uint16_t* m, int rs, int r0, int c0, int lane) {
    const int g = lane >> 4, a = lane & 15;
    const uint16_t* p = m + (r0 + 8 * g + (a >> 2)) * rs + npos(c0 + 4 * (a & 3));
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

// One thread's share of a chunk's inputs, fetched a chunk ahead: token
// tid / 8 and an eighth of its x, z, B and C rows; wave 4 (which runs the
// decay prefix) also Delta of token lane.
template <int N>
struct ChunkRegs {
    static constexpr int kBC = N / 64;   // 16-byte pieces of an eighth of a B (or C) row
    u32x4 x, z;
    u32x4 b[kBC], c[kBC];
    unsigned short dt;
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
    float Y[2][kQ][kRowY];        // each n-half's 2^cum C S (+ its share of M X), [t][p]
    float dl[2][kQ];              // Delta, by chunk parity
    float cum[2][kQ];             // inclusive prefix of w A within the chunk
    float wts[2][kQ];             // 2^(cum_last - cum_s) Delta_s
    float ecum[2][kQ];            // 2^cum_t
};

// The causal 16 x 16 tiles (t-tile, s-tile) of M; wave w builds tiles w and
// w + 8.  Tiles (0, 1) and (2, 3) lie above the diagonal but inside the
// 32-wide k-steps of M X: they stay zero.
__device__ __forceinline__ void m_tile(int k, int& tb, int& sb) {
    tb = k >= 6 ? 3 : k >= 3 ? 2 : k >= 1 ? 1 : 0;
    sb = k - tb * (tb + 1) / 2;
}

// Per chunk (barriers between phases), every wave:
//   B  Y_half = 2^cum C S over its n-half and 16 columns; M tiles
//   C  its t-tiles of M X added, Y_half to LDS; its piece of the weighted x;
//      silu(z) and D x silu(z) of its 8 outputs (wave 4: the next prefix)
//   D  y of its 8 outputs = (Y_0 + Y_1) silu(z) + D x silu(z), stored;
//      S = 2^cum_last S + B^T (w X) for its tiles, and their split
//   A  its piece of the next chunk into LDS; the one after requested
template <typename Tout, int N, bool SP>
__global__ __launch_bounds__(kThreads) void m2_ssd_kernel(M2Args a) {
    constexpr int NH = N / 2;                // state rows per wave
    constexpr int NT = NH / 16;              // 16-row state tiles per wave
    constexpr int KS = NH / 32;              // k-steps of C S per wave
    constexpr int NBC = ChunkRegs<N>::kBC;
    constexpr int kRowN = SsdSmem<N>::kRowN;
    __shared__ __attribute__((aligned(16))) SsdSmem<N> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 15;                // MFMA column / row within a 16-tile
    const int lg = lane >> 4;                // lane group: k offset 8 lg, output rows 4 lg + q
    const int nh = wave >> 2;                // n-half of the wave's state rows
    const int nb0 = NH * nh;
    const int pq = wave & 3;                 // the wave's 16 state columns
    const int pcol = 16 * pq + li;
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
    // byte strides of one token
    const int64_t sx = H * kPd * 2, sbc = G * N * 2, sd = H * 2, sy = H * kPd * (int64_t)sizeof(Tout);

    // state tile j: rows n = nb0 + 16 j + 4 lg + q, column pcol
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
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            S[j][q] = a.h0 ? a.h0[(bh * kPd + pcol) * N + nb0 + 16 * j + 4 * lg + q] : 0.0f;
    split_state();

    const int64_t nch = (L + kQ - 1) / kQ;
    const int rt = tid >> 3, rq = tid & 7;   // staging and output: token, eighth of a row
    // The chunk at t0 through descriptors bounded at token L - 1 (past it:
    // zeros).  Issued for every chunk, also the one past the end.
    auto fetch = [&](int64_t t0, ChunkRegs<N>& r) {
        const int64_t rows = L - t0 < kQ ? L - t0 : kQ;
        if (wave == 4) {
            const auto rd = rows_rsrc(DT + (b * L + t0) * H + h, rows, sd, 2);
            r.dt = __builtin_amdgcn_raw_buffer_load_b16(rd, (int)(lane * sd), 0, 0);
        }
        const int64_t xo = ((b * L + t0) * H + h) * kPd;
        const auto rx = rows_rsrc(X + xo, rows, sx, kPd * 2);
        r.x = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(rt * sx) + 16 * rq, 0, 0);
        if (Z) {
            const auto rz = rows_rsrc(Z + xo, rows, sx, kPd * 2);
            r.z = __builtin_amdgcn_raw_buffer_load_b128(rz, (int)(rt * sx) + 16 * rq, 0, 0);
        }
        const int64_t bo = ((b * L + t0) * G + grp) * N;
        const auto rb = rows_rsrc(Bg + bo, rows, sbc, N * 2);
        const auto rc = rows_rsrc(Cg + bo, rows, sbc, N * 2);
#pragma unroll
        for (int q = 0; q < NBC; ++q) {
            r.b[q] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(rt * sbc) + 16 * (NBC * rq + q), 0, 0);
            r.c[q] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(rt * sbc) + 16 * (NBC * rq + q), 0, 0);
        }
    };
    // Delta, the in-chunk prefix of the log2 decay and the per-token factors
    // of the chunk at t0 (tokens past L: Delta 0, decay 1, no input)
    auto prefix = [&](int64_t t0, unsigned short dt, int buf) {
        float wv = 0.0f;
        if (t0 + lane < L) {
            const float vl = __builtin_fmaf(bf16_to_f32(dt), kLog2e, bias_l);
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

    // this thread's piece of a chunk into LDS
    auto stage = [&](const ChunkRegs<N>& r) {
        *reinterpret_cast<u32x4*>(&sm.xs[rt][8 * rq]) = r.x;
        *reinterpret_cast<u32x4*>(&sm.zs[rt][8 * rq]) = r.z;
#pragma unroll
        for (int q = 0; q < NBC; ++q) {
            const int n0 = 8 * (NBC * rq + q);
            *reinterpret_cast<uint2*>(&sm.Bs[rt][npos(n0)]) = make_uint2(r.b[q].x, r.b[q].y);
            *reinterpret_cast<uint2*>(&sm.Bs[rt][npos(n0 + 4)]) = make_uint2(r.b[q].z, r.b[q].w);
            *reinterpret_cast<uint2*>(&sm.Cs[rt][npos(n0)]) = make_uint2(r.c[q].x, r.c[q].y);
            *reinterpret_cast<uint2*>(&sm.Cs[rt][npos(n0 + 4)]) = make_uint2(r.c[q].z, r.c[q].w);
        }
    };

    // Chunk 0 is staged here and every iteration ends by staging the next
    // one, so the chunk's loads are always followed by exactly the y stores
    // of one chunk: the wait at the staging then never includes those stores.
    ChunkRegs<N> cr;
    cr.z = u32x4{0u, 0u, 0u, 0u};
    fetch(0, cr);
    if (wave == 4) prefix(0, cr.dt, 0);
    stage(cr);
    fetch(kQ, cr);
    if (tid < 256) {
        // the zero tiles of M, written once: one 16-byte piece per even
        // thread of tile (0, 1) or (2, 3), hi or lo
        const int tile = tid >> 7, hl = (tid >> 6) & 1, r = (tid >> 2) & 15, c8 = (tid >> 1) & 1;
        if ((tid & 1) == 0) {
            const int t = 32 * tile + r, s = 32 * tile + 16 + 8 * c8;
            uint16_t* dst = hl ? &sm.Ml[t][s] : &sm.Mh[t][s];
            *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
        }
    }
    lds_barrier();

    float eg[8], edg[8];   // silu(z) and D x silu(z) of the thread's outputs, from phase C to D

    for (int64_t c = 0; c < nch; ++c) {
        const int64_t t0 = c * kQ;
        const int cb = (int)(c & 1);
        // ---- B: 2^cum C S over the wave's n-half; M tiles ------------------
        // k-step ks pairs state tiles 2 ks and 2 ks + 1, whose rows
        // 4 lg .. 4 lg + 3 this lane holds: the C operand takes columns
        // nb0 + 32 ks + 4 lg .. + 3 and nb0 + 32 ks + 16 + 4 lg .. + 3
        f32x4 Yacc[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            Yacc[tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            const uint16_t* crow = &sm.Cs[16 * tb + li][nb0 + 8 * lg];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 cv = ld8(crow + 32 * ks);
                Yacc[tb] = mfma(cv, Sh[ks], Yacc[tb]);
                Yacc[tb] = mfma(cv, Sl[ks], Yacc[tb]);
            }
            Yacc[tb] *= *reinterpret_cast<const f32x4*>(&sm.ecum[cb][16 * tb + 4 * lg]);
        }
        for (int k = wave; k < 10; k += kWaves) {
            int tb, sb;
            m_tile(k, tb, sb);
            // M^T tile = B C^T: rows s = 16 sb + 4 lg + q, column t = 16 tb + li
            f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < N / 32; ++ks)
                g = mfma(ld8(&sm.Bs[16 * sb + li][32 * ks + 8 * lg]), ld8(&sm.Cs[16 * tb + li][32 * ks + 8 * lg]), g);
            const int t = 16 * tb + li, s0 = 16 * sb + 4 * lg;
            const float ct = sm.cum[cb][t];
            const f32x4 cs = *reinterpret_cast<const f32x4*>(&sm.cum[cb][s0]);
            const f32x4 ds = *reinterpret_cast<const f32x4*>(&sm.dl[cb][s0]);
            float m[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) m[q] = (s0 + q <= t) ? g[q] * fast_exp2(ct - cs[q]) * ds[q] : 0.0f;
            uint2 mh, ml;
            split4(m, mh, ml);
            *reinterpret_cast<uint2*>(&sm.Mh[t][s0]) = mh;
            *reinterpret_cast<uint2*>(&sm.Ml[t][s0]) = ml;
        }
        lds_barrier();

        // ---- C: M X for the wave's t-tiles, Y_half to LDS; weighted x; gate -
        // n-half 0 takes t-tiles 0 and 3, n-half 1 t-tiles 1 and 2 (six
        // MFMAs each: t-tiles 2 and 3 span both 32-token k-steps)
        // (the t-tiles are compile-time constants in each branch, so Yacc
        // stays in fixed registers)
        auto mx = [&](auto tbc) {
            constexpr int tb = decltype(tbc)::value;
#pragma unroll
            for (int ks = 0; ks <= (tb >> 1); ++ks) {
                const bf16x8 xv = ld_col8(&sm.xs[0][0], kRowX, 32 * ks, 16 * pq, lane);
                Yacc[tb] = mfma(ld8(&sm.Mh[16 * tb + li][32 * ks + 8 * lg]), xv, Yacc[tb]);
                Yacc[tb] = mfma(ld8(&sm.Ml[16 * tb + li][32 * ks + 8 * lg]), xv, Yacc[tb]);
            }
        };
        if (nh == 0) {
            mx(std::integral_constant<int, 0>{});
            mx(std::integral_constant<int, 3>{});
        } else {
            mx(std::integral_constant<int, 1>{});
            mx(std::integral_constant<int, 2>{});
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int q = 0; q < 4; ++q) sm.Y[nh][16 * tb + 4 * lg + q][pcol] = Yacc[tb][q];
        {
            const float wv = sm.wts[cb][rt];
            const bf16x8 xv = ld8(&sm.xs[rt][8 * rq]);
            const bf16x8 zv = ld8(&sm.zs[rt][8 * rq]);
            bf16x8 xh, xl;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = (float)xv[j];
                const float v = x * wv;
                const __bf16 vh = (__bf16)v;
                xh[j] = vh;
                xl[j] = (__bf16)(v - (float)vh);
                const float gz = Z ? silu_scaled((float)zv[j], 1.0f) : 1.0f;
                eg[j] = gz;
                edg[j] = Dh * x * gz;
            }
            *reinterpret_cast<bf16x8*>(&sm.Wh[rt][8 * rq]) = xh;
            *reinterpret_cast<bf16x8*>(&sm.Wl[rt][8 * rq]) = xl;
        }
        // the next chunk's prefix (cr holds chunk c + 1)
        if (wave == 4 && c + 1 < nch) prefix(t0 + kQ, cr.dt, cb ^ 1);
        lds_barrier();

        // ---- D: y of the thread's 8 outputs; the state update --------------
        {
            float yv[8];
#pragma unroll
            for (int j4 = 0; j4 < 2; ++j4) {
                const f32x4 y0 = *reinterpret_cast<const f32x4*>(&sm.Y[0][rt][8 * rq + 4 * j4]);
                const f32x4 y1 = *reinterpret_cast<const f32x4*>(&sm.Y[1][rt][8 * rq + 4 * j4]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    yv[4 * j4 + q] = __builtin_fmaf(y0[q] + y1[q], eg[4 * j4 + q], edg[4 * j4 + q]);
            }
            const int64_t rows = L - t0 < kQ ? L - t0 : kQ;
            const auto ry = rows_rsrc(Yg + ((b * L + t0) * H + h) * kPd, rows, sy, kPd * (int)sizeof(Tout));
            const int yo = (int)(rt * sy) + 8 * rq * (int)sizeof(Tout);
            if constexpr (sizeof(Tout) == 4) {
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(yv[0]), __float_as_uint(yv[1]),
                                                             __float_as_uint(yv[2]), __float_as_uint(yv[3])},
                                                       ry, yo, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(yv[4]), __float_as_uint(yv[5]),
                                                             __float_as_uint(yv[6]), __float_as_uint(yv[7])},
                                                       ry, yo + 16, 0, 0);
            } else {
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]),
                                                             pack_bf16x2(yv[4], yv[5]), pack_bf16x2(yv[6], yv[7])},
                                                       ry, yo, 0, 0);
            }
        }
        {
            const float dec = sm.ecum[cb][kQ - 1];
#pragma unroll
            for (int j = 0; j < NT; ++j) S[j] *= dec;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 wh = ld_col8(&sm.Wh[0][0], kRowX, 32 * ks, 16 * pq, lane);
                const bf16x8 wl = ld_col8(&sm.Wl[0][0], kRowX, 32 * ks, 16 * pq, lane);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    // B^T operand: row n = nb0 + 16 j + li, k = s
                    const bf16x8 bt = ld_col8_n(&sm.Bs[0][0], kRowN, 32 * ks, nb0 + 16 * j, lane);
                    S[j] = mfma(bt, wh, S[j]);
                    S[j] = mfma(bt, wl, S[j]);
                }
            }
            split_state();
        }
        lds_barrier();

        // ---- A: stage the next chunk; request the one after ----------------
        stage(cr);
        fetch(t0 + 2 * kQ, cr);
        lds_barrier();
    }

    if (a.last) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) a.last[(bh * kPd + pcol) * N + nb0 + 16 * j + 4 * lg + q] = S[j][q];
    }
}

// ---------------------------------------------------------------------------
// Warp-specialised form.  Waves 0..3 ("state waves") each hold the state of
// one 16-column p-tile for every n; per chunk they compute 2^cum C S, the gate
// silu(z) and D x silu(z) of their outputs, y of the chunk before (adding the
// chunk waves' M X), and the state update, with the weighted x built on the
// fly from x and the decay weights.  Waves 4..7 ("chunk waves") each own one
// 16-token t-tile: they build their rows of M in registers (no LDS round
// trip) and M X, and stage the inputs.  The two groups meet at one barrier
// per chunk: in iteration c the state waves finish y of chunk c - 1 and work
// on chunk c while the chunk waves compute M X of chunk c and stage chunk
// c + 1.  Every LDS array the groups exchange is double-buffered by chunk
// parity, so the matrix-core work of one group overlaps the vector and LDS
// work of the other instead of all waves running the same phase at once.
// The state waves' path is the longer one; the gate still sits with them,
// because staged from the chunk waves (as silu(z) in fp32) it made the chunk
// wave of t-tile 3, which carries the largest share of M (four 16x16 tiles
// against one for t-tile 0), the slower side of the barrier.
//
// Both groups work in the transposed orientation where that puts a lane's
// values in the layout its consumer needs: C S and M X are computed as
// (S^T C^T) and (X^T M^T), whose accumulators give each lane one token and
// four consecutive channels p, the row-major order of y.

// MFMA operand with k running down a row-major matrix in the permuted order
// of an accumulator's rows: lane l = 16 g + i gets rows r0 + 4 g .. + 3, then
// r0 + 16 + 4 g .. + 3, of column c0 + i (k-step over two 16-row tiles).
__device__ __forceinline__ bf16x8 ld_col8_acc(const uint16_t* m, int rs, int r0, int c0, int lane) {
    const int g = lane >> 4, a = lane & 15;
    const uint16_t* p = m + (r0 + 4 * g + (a >> 2)) * rs + c0 + 4 * (a & 3);
    return cat(ld_tr(p), ld_tr(p + 16 * rs));
}

// bf16 hi + lo halves of two fp32 values as packed pairs (hi = bf16(v),
// lo = bf16(v - hi)): one conversion per pair rather than one per value.
__device__ __forceinline__ void split2(float a, float b, unsigned& hi, unsigned& lo) {
    hi = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - bf16lo(hi), b - bf16hi(hi));
}

// Eight fp32 values split into two MFMA operands (k order kept).
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
    unsigned h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(v[2 * i], v[2 * i + 1], h[i], l[i]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

template <int N>
struct WsSmem {
    // B and C rows padded by 16 elements (a stride of 8 banks mod 32): the
    // transposed B reads of the state update, four consecutive rows per lane
    // group, then fall in distinct banks (measured: 4 % less time than a
    // padding of 8, which suits only the row-wise reads)
    static constexpr int kRowN = N + 16;
    uint16_t Bs[2][kQ][kRowN];    // B, [s][n] (n permuted by npos)
    uint16_t Cs[2][kQ][kRowN];    // C, [t][n] (n permuted by npos)
    uint16_t xs[2][kQ][kRowX];    // x, [s][p]
    uint16_t zs[2][kQ][kRowX];    // z, [t][p]
    float Yc[2][kQ][kRowY];       // M X of the chunk, [t][p]
    float dl[2][kQ];              // Delta
    float cum[2][kQ];             // inclusive prefix of w A within the chunk
    float wts[2][kQ];             // 2^(cum_last - cum_s) Delta_s
    float ecum[2][kQ];            // 2^cum_t
};

// A chunk wave thread's quarter of one token's inputs, fetched a chunk ahead.
template <int N>
struct WsRegs {
    static constexpr int kBC = N / 32;   // 16-byte pieces of a quarter B (or C) row
    u32x4 x[2], z[2];
    u32x4 b[kBC], c[kBC];
    unsigned short dt;
};

template <typename Tout, int N, bool SP>
__global__ __launch_bounds__(kThreads) void m2_ssd_ws_kernel(M2Args a) {
    constexpr int NT = N / 16;               // 16-row state tiles per state wave
    constexpr int KS = N / 32;               // k-steps over n
    constexpr int NBC = WsRegs<N>::kBC;
    constexpr int kRowN = WsSmem<N>::kRowN;
    __shared__ __attribute__((aligned(16))) WsSmem<N> sm;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the roles branch on it
    const int lane = tid & 63;
    const int li = lane & 15;
    const int lg = lane >> 4;
    // (batch, head) unit: workgroups are dealt to the 8 XCDs round-robin by
    // id, so unit id % 8 * (units / 8) + id / 8 puts consecutive units, the
    // heads of one batch that share its B and C, on one XCD and its L2
    const int64_t nbh = a.batch * a.H;
    const int64_t bh = (a.xcd_units && nbh % 8 == 0) ? (int64_t)(blockIdx.x % 8) * (nbh / 8) + blockIdx.x / 8
                                                     : (int64_t)blockIdx.x;
    const int64_t b = bh / a.H;
    const int64_t h = bh - b * a.H;
    const int64_t grp = h / (a.H / a.G);
    const int64_t L = a.L;
    const int64_t H = a.H, G = a.G;
    const int64_t nch = (L + kQ - 1) / kQ;
    const uint16_t* Z = reinterpret_cast<const uint16_t*>(a.z);

    if (wave < 4) {
        // ---------------- state waves: p-tile `wave`, every n ----------------
        // A lane's outputs: token 16 tb + li, channels 16 pt + 4 lg .. + 3,
        // for the four t-tiles tb.
        const int pt = wave;
        const int pcol = 16 * pt + li;
        // 1 and 0 with a gate, 0 and 1 without; opaque, so that the blend
        // below stays arithmetic (a select per value becomes a branch)
        float zon = Z != nullptr ? 1.0f : 0.0f;
        asm volatile("" : "+v"(zon));
        const float zoff = 1.0f - zon;
        const float Dh = a.D ? a.D[h] : 0.0f;
        Tout* Yg = reinterpret_cast<Tout*>(a.y);
        const int64_t sy = H * kPd * (int64_t)sizeof(Tout);
        // state tile j: rows n = 16 j + 4 lg + q, column pcol
        f32x4 S[NT];
        bf16x8 Sh[KS], Sl[KS];   // S^T as A operands (k-step ks: tiles 2 ks, 2 ks + 1)
        auto split_state = [&]() {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const float v[8] = {S[2 * ks][0],     S[2 * ks][1],     S[2 * ks][2],     S[2 * ks][3],
                                    S[2 * ks + 1][0], S[2 * ks + 1][1], S[2 * ks + 1][2], S[2 * ks + 1][3]};
                split8(v, Sh[ks], Sl[ks]);
            }
        };
        // chunk c - 1 carried across the barrier: 2^cum C S, silu(z), D x silu(z)
        f32x4 Ye[4];
        float eg[16], edg[16];
        // y of chunk c (M X from buffer cb), for c = -1 too through an empty
        // descriptor that drops the stores
        auto fin = [&](int64_t c, int cb) {
            const int64_t t0 = c * kQ;
            const int64_t rows = c < 0 ? 0 : L - t0 < kQ ? L - t0 : kQ;
            const auto ry = rows_rsrc(Yg + ((b * L + t0) * H + h) * kPd, rows, sy, kPd * (int)sizeof(Tout));
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + li;
                const f32x4 yi = *reinterpret_cast<const f32x4*>(&sm.Yc[cb][t][16 * pt + 4 * lg]);
                float yv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    yv[q] = __builtin_fmaf(yi[q] + Ye[tb][q], eg[4 * tb + q], edg[4 * tb + q]);
                const int yo = (int)(t * sy) + (16 * pt + 4 * lg) * (int)sizeof(Tout);
                if constexpr (sizeof(Tout) == 4) {
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(yv[0]), __float_as_uint(yv[1]),
                                                                 __float_as_uint(yv[2]), __float_as_uint(yv[3])},
                                                           ry, yo, 0, 0);
                } else {
                    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])}, ry, yo, 0, 0);
                }
            }
        };
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                S[j][q] = a.h0 ? a.h0[(bh * kPd + pcol) * N + 16 * j + 4 * lg + q] : 0.0f;
        split_state();
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) Ye[tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 16; ++i) eg[i] = edg[i] = 0.0f;
        lds_barrier();   // chunk 0 staged

        for (int64_t c = 0; c < nch; ++c) {
            const int cb = (int)(c & 1);
            fin(c - 1, cb ^ 1);
            // (S^T C^T)[p, t] 2^cum_t for each t-tile
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
                const uint16_t* crow = &sm.Cs[cb][16 * tb + li][8 * lg];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 cv = ld8(crow + 32 * ks);
                    acc = mfma(Sh[ks], cv, acc);
                    acc = mfma(Sl[ks], cv, acc);
                }
                Ye[tb] = acc * sm.ecum[cb][16 * tb + li];
            }
            // the gate of the lane's outputs
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + li;
                const uint2 xw = *reinterpret_cast<const uint2*>(&sm.xs[cb][t][16 * pt + 4 * lg]);
                const uint2 zw = *reinterpret_cast<const uint2*>(&sm.zs[cb][t][16 * pt + 4 * lg]);
                const float xq[4] = {bf16lo(xw.x), bf16hi(xw.x), bf16lo(xw.y), bf16hi(xw.y)};
                const float zq[4] = {bf16lo(zw.x), bf16hi(zw.x), bf16lo(zw.y), bf16hi(zw.y)};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // gate = silu(z), or 1 without z (z is staged as zeros,
                    // silu(0) = 0): a blend rather than a branch per value
                    const float gz = __builtin_fmaf(silu_scaled(zq[q], 1.0f), zon, zoff);
                    eg[4 * tb + q] = gz;
                    edg[4 * tb + q] = Dh * xq[q] * gz;
                }
            }
            // S = 2^cum_last S + B^T diag(w) X, the weighted x split as it is read
            const float dec = sm.ecum[cb][kQ - 1];
#pragma unroll
            for (int j = 0; j < NT; ++j) S[j] *= dec;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 xv = ld_col8(&sm.xs[cb][0][0], kRowX, 32 * ks, 16 * pt, lane);
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sm.wts[cb][32 * ks + 8 * lg]);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sm.wts[cb][32 * ks + 8 * lg + 4]);
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = (float)xv[j] * (j < 4 ? w0[j] : w1[j - 4]);
                bf16x8 wh, wl;
                split8(v, wh, wl);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    // B^T operand: row n = 16 j + li, k = s
                    const bf16x8 bt = ld_col8_n(&sm.Bs[cb][0][0], kRowN, 32 * ks, 16 * j, lane);
                    S[j] = mfma(bt, wh, S[j]);
                    S[j] = mfma(bt, wl, S[j]);
                }
            }
            split_state();
            lds_barrier();
        }
        fin(nch - 1, (int)((nch - 1) & 1));
        if (a.last) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) a.last[(bh * kPd + pcol) * N + 16 * j + 4 * lg + q] = S[j][q];
        }
        return;
    }

    // ---------------- chunk waves: t-tile `wave - 4` --------------------------
    const int tb = wave - 4;
    const int t = 16 * tb + li;              // this lane's token within a chunk
    // issue priority over the state wave sharing the SIMD (measured: about
    // 1.5 % less time)
    __builtin_amdgcn_s_setprio(3);
    const int ct = tid - 256;
    const int rt = ct >> 2, rq = ct & 3;     // staging: token, quarter of a row
    const float Ah = a.A[h];
    const float bias_l = (a.dt_bias ? a.dt_bias[h] : 0.0f) * kLog2e;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x);
    const uint16_t* DT = reinterpret_cast<const uint16_t*>(a.dt);
    const uint16_t* Bg = reinterpret_cast<const uint16_t*>(a.B);
    const uint16_t* Cg = reinterpret_cast<const uint16_t*>(a.C);
    const int64_t sx = H * kPd * 2, sbc = G * N * 2, sd = H * 2;

    auto fetch = [&](int64_t t0, WsRegs<N>& r) {
        const int64_t rows = L - t0 < kQ ? L - t0 : kQ;
        if (wave == 4) {
            const auto rd = rows_rsrc(DT + (b * L + t0) * H + h, rows, sd, 2);
            r.dt = __builtin_amdgcn_raw_buffer_load_b16(rd, (int)(lane * sd), 0, 0);
        }
        const int64_t xo = ((b * L + t0) * H + h) * kPd;
        const auto rx = rows_rsrc(X + xo, rows, sx, kPd * 2);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            r.x[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(rt * sx) + 32 * rq + 16 * i, 0, 0);
        if (Z) {
            const auto rz = rows_rsrc(Z + xo, rows, sx, kPd * 2);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                r.z[i] = __builtin_amdgcn_raw_buffer_load_b128(rz, (int)(rt * sx) + 32 * rq + 16 * i, 0, 0);
        }
        const int64_t bo = ((b * L + t0) * G + grp) * N;
        const auto rb = rows_rsrc(Bg + bo, rows, sbc, N * 2);
        const auto rc = rows_rsrc(Cg + bo, rows, sbc, N * 2);
#pragma unroll
        for (int q = 0; q < NBC; ++q) {
            r.b[q] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(rt * sbc) + 16 * (NBC * rq + q), 0, 0);
            r.c[q] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(rt * sbc) + 16 * (NBC * rq + q), 0, 0);
        }
    };
    // Delta, the in-chunk prefix of the log2 decay and the per-token factors
    // of the chunk at t0 (tokens past L: Delta 0, decay 1, no input)
    auto prefix = [&](int64_t t0, unsigned short dt, int buf) {
        float wv = 0.0f;
        if (t0 + lane < L) {
            const float vl = __builtin_fmaf(bf16_to_f32(dt), kLog2e, bias_l);
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
    auto stage = [&](const WsRegs<N>& r, int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            *reinterpret_cast<u32x4*>(&sm.xs[buf][rt][16 * rq + 8 * i]) = r.x[i];
            *reinterpret_cast<u32x4*>(&sm.zs[buf][rt][16 * rq + 8 * i]) = r.z[i];
        }
#pragma unroll
        for (int q = 0; q < NBC; ++q) {
            const int n0 = 8 * (NBC * rq + q);
            *reinterpret_cast<uint2*>(&sm.Bs[buf][rt][npos(n0)]) = make_uint2(r.b[q].x, r.b[q].y);
            *reinterpret_cast<uint2*>(&sm.Bs[buf][rt][npos(n0 + 4)]) = make_uint2(r.b[q].z, r.b[q].w);
            *reinterpret_cast<uint2*>(&sm.Cs[buf][rt][npos(n0)]) = make_uint2(r.c[q].x, r.c[q].y);
            *reinterpret_cast<uint2*>(&sm.Cs[buf][rt][npos(n0 + 4)]) = make_uint2(r.c[q].z, r.c[q].w);
        }
    };

    // (X^T M^T)[p, t] of chunk buffer cb for t-tile TB, into Yc.  The rows of
    // M^T come from the MFMA (B C^T) in the accumulator layout (lane: column
    // t, rows s = 16 sb + 4 lg + q), which is the B operand of the product with
    // k = s permuted to match; X^T is read in the same order.
    auto prep = [&](auto tbc, int cb) {
        constexpr int TB = decltype(tbc)::value;
        constexpr int KX = TB / 2 + 1;   // 32-token k-steps of M X
        bf16x8 cop[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) cop[ks] = ld8(&sm.Cs[cb][t][32 * ks + 8 * lg]);
        const float ctv = sm.cum[cb][t];
        unsigned mh[KX][4], ml[KX][4];   // bf16 pairs: words 2 (sb & 1), + 1 of k-step sb / 2
#pragma unroll
        for (int sb = 0; sb < 2 * KX; ++sb) {
            float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (sb <= TB) {
                f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) g = mfma(ld8(&sm.Bs[cb][16 * sb + li][32 * ks + 8 * lg]), cop[ks], g);
                const int s0 = 16 * sb + 4 * lg;
                const f32x4 cs = *reinterpret_cast<const f32x4*>(&sm.cum[cb][s0]);
                const f32x4 ds = *reinterpret_cast<const f32x4*>(&sm.dl[cb][s0]);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    m[q] = (sb < TB || s0 + q <= t) ? g[q] * fast_exp2(ctv - cs[q]) * ds[q] : 0.0f;
            }
#pragma unroll
            for (int q = 0; q < 2; ++q)
                split2(m[2 * q], m[2 * q + 1], mh[sb >> 1][2 * (sb & 1) + q], ml[sb >> 1][2 * (sb & 1) + q]);
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            f32x4 yi = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KX; ++ks) {
                const bf16x8 xa = ld_col8_acc(&sm.xs[cb][0][0], kRowX, 32 * ks, 16 * pt, lane);
                yi = mfma(xa, __builtin_bit_cast(bf16x8, u32x4{mh[ks][0], mh[ks][1], mh[ks][2], mh[ks][3]}), yi);
                yi = mfma(xa, __builtin_bit_cast(bf16x8, u32x4{ml[ks][0], ml[ks][1], ml[ks][2], ml[ks][3]}), yi);
            }
            *reinterpret_cast<f32x4*>(&sm.Yc[cb][t][16 * pt + 4 * lg]) = yi;
        }
    };

    WsRegs<N> cr;
    cr.z[0] = cr.z[1] = u32x4{0u, 0u, 0u, 0u};
    fetch(0, cr);
    if (wave == 4) prefix(0, cr.dt, 0);
    stage(cr, 0);
    fetch(kQ, cr);
    lds_barrier();

    for (int64_t c = 0; c < nch; ++c) {
        const int64_t t0 = c * kQ;
        const int cb = (int)(c & 1);
        switch (tb) {
            case 0: prep(std::integral_constant<int, 0>{}, cb); break;
            case 1: prep(std::integral_constant<int, 1>{}, cb); break;
            case 2: prep(std::integral_constant<int, 2>{}, cb); break;
            default: prep(std::integral_constant<int, 3>{}, cb); break;
        }
        // chunk c + 1 into the other buffer (its prefix from wave 4), then
        // request chunk c + 2
        stage(cr, cb ^ 1);
        if (wave == 4 && c + 1 < nch) prefix(t0 + kQ, cr.dt, cb ^ 1);
        fetch(t0 + 2 * kQ, cr);
        lds_barrier();
    }
}

template <typename Tout, int N>
hipError_t launch_n(const M2Args& a, int ws, hipStream_t stream) {
    const unsigned blocks = (unsigned)(a.batch * a.H);
    KTime kt("m2_ssd", stream);
    if (ws) {
        if (a.softplus)
            hipLaunchKernelGGL((m2_ssd_ws_kernel<Tout, N, true>), dim3(blocks), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((m2_ssd_ws_kernel<Tout, N, false>), dim3(blocks), dim3(kThreads), 0, stream, a);
    } else if (a.softplus) {
        hipLaunchKernelGGL((m2_ssd_kernel<Tout, N, true>), dim3(blocks), dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL((m2_ssd_kernel<Tout, N, false>), dim3(blocks), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

// The buffer descriptors hold 32-bit byte counts and offsets: one chunk of
// 64 tokens of x or y (or of B) must span less than 2 GB.
bool m2_ssd_supported(const M2Args& a, int in_bf16) {
    const int64_t chunk_x = kQ * a.H * a.P * 4, chunk_b = kQ * a.G * a.N * 2;
    return in_bf16 && a.P == kPd && (a.N == 64 || a.N == 128) && a.batch * a.H < 0x7fffffff &&
           chunk_x < (int64_t(1) << 31) && chunk_b < (int64_t(1) << 31);
}

hipError_t launch_m2_ssd(const M2Args& a, int out_bf16, int ws, hipStream_t stream) {
    if (a.N == 128) return out_bf16 ? launch_n<uint16_t, 128>(a, ws, stream) : launch_n<float, 128>(a, ws, stream);
    return out_bf16 ? launch_n<uint16_t, 64>(a, ws, stream) : launch_n<float, 64>(a, ws, stream);
}

}  // namespace selscan
