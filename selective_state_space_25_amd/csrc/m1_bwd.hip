// m1_bwd.hip -- gradients of the Mamba-1 selective scan for gfx950.
//
// Reverse mode through the recurrence of section 2.2 of the "Understanding
// Mamba and Selective State Space Models (SSMs)" blog (the training side of
// the README's selective SSM layer).  With a_t[n] = exp(Delta_t A[n]),
// out_t = y_t silu(z_t) and dout given, the state's adjoint runs backward:
//
//   dy_t     = dout_t silu(z_t)
//   lam_t[n] = dy_t C_t[n] + a_{t+1}[n] lam_{t+1}[n]
//   dC_t[n]  = sum_d dy_t h_t[n]        dB_t[n] = sum_d lam_t[n] Delta_t u_t
//   du_t     = dy_t D + Delta_t sum_n lam_t[n] B_t[n]
//   dDelta_t = sum_n lam_t[n] (B_t[n] u_t + A[n] a_t[n] h_{t-1}[n])
//   dA[n]    = sum_{b,t} Delta_t lam_t[n] a_t[n] h_{t-1}[n]
//
// Time is cut into chunks so that the grid fills the chip:
//   summary: per chunk, a forward sweep from a zero state that stores the
//            state (and the running sum of Delta) every 16 tokens and the
//            state at the chunk's end; and a reverse sweep of the adjoint from
//            a zero right boundary;
//   carry:   the true state entering each chunk (forward over chunks, from
//            h0) and the true adjoint entering it from the right (backward
//            over chunks); both are linear, so a chunk's decay
//            exp(A sum Delta) is all that links neighbours;
//   chunk:   per chunk, 16-token tiles from the last: the tile's first state
//            is the stored zero-start state plus the decayed entering state;
//            the tile's 16 states are recomputed into registers and the
//            adjoint runs back through them;
//   reduce:  sums of the per-block partials over channel blocks, batches and
//            chunks (no atomics: results do not depend on scheduling).
//
// A workgroup is 256 threads for 64 channels of one batch.  A lane holds 4 of
// a channel's 16 states (n = 4q .. 4q+3); lane = 16 dr + 4 q + rr, channel =
// 16 wave + 4 dr + rr.  Per-channel, per-token values (Delta, Delta u, dy, ...)
// are computed once per tile by a "producer" mapping (thread = channel x 4
// tokens) into LDS.  Sums over n go over a lane's 4 states and then across
// the 4 lanes of the channel (DPP row rotations by 4 and 8); dB and dC, sums
// over channels, are reduce-scattered across the 4 channels of a DPP row
// (quad permutes), then across the wave's 4 DPP rows (permlane32/16 swaps),
// then across the 4 waves in LDS.
#include "device_math.hpp"
#include "kernels.hpp"
#include "lds_rows.hpp"

namespace selscan {

namespace {

constexpr int kCh = 64;          // channels per workgroup
constexpr int kSt = 16;          // states per channel (padded)
constexpr int kT = 16;           // tokens per tile (16 rather than 8: half the requests per token)
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPad = kT + 1;     // LDS row pitch of per-channel tile values
constexpr int kPT = kT / 4;      // tokens per producer thread (4 threads per channel)
constexpr int kRT = 256 / (2 * kSt);   // tokens per 256-thread dB/dC partial pass

template <typename T> __device__ __forceinline__ float ld1(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld1<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

// v + v of another lane, by a DPP control (row rotations, quad permutes)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kRor4 = 0x124, kRor8 = 0x128, kQuadX1 = 0xB1, kQuadX2 = 0x4E;

// sum over the 4 lanes of a channel (lanes 4 apart in a DPP row)
__device__ __forceinline__ float sum_q(float v) {
    v += dpp<kRor4>(v);
    return v + dpp<kRor8>(v);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its global loads (prefetches stay in flight) or stores.
// No data passes between threads through global memory inside a kernel here.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float sigmoid(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }

// Delta = softplus(x) (natural units) and its derivative sigmoid(x)
template <bool SP>
__device__ __forceinline__ float delta_of(float x, float& deriv) {
    if (!SP) {
        deriv = 1.0f;
        return x;
    }
    const float e = fast_exp2(-fabsf(x) * kLog2e);       // exp(-|x|) in (0, 1]
    const float r = fast_rcp(1.0f + e);
    deriv = x >= 0.0f ? r : e * r;
    return softplus_log2(x * kLog2e) * kLn2;
}

// Uniform per workgroup: its (batch, channel block, chunk) and the first row
// of its channel block.  Tensors are addressed from per-workgroup base
// pointers (scalar registers) with 32-bit per-thread byte offsets, which the
// hardware adds to the base itself; the host keeps L <= 2^22, so every byte
// offset within a workgroup's rows fits in 32 bits.
// element idx of base through a 32-bit byte offset
template <typename T>
__device__ __forceinline__ T ldo(const T* base, uint32_t idx) {
    return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + idx * (uint32_t)sizeof(T));
}
template <typename T>
__device__ __forceinline__ void sto(T* base, uint32_t idx, T v) {
    *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + idx * (uint32_t)sizeof(T)) = v;
}

// Stores inside the tile loops go through a buffer descriptor spanning the
// block's part of the output; a lane that must not store passes the span's
// end as its offset, and the hardware drops out-of-range stores.  Every lane
// thus issues the same stores with no branch around them: after a branch the
// compiler cannot count the stores in flight and waits for all of them
// before the next tile's prefetched loads are used.
constexpr int kBufWord3 = 0x00020000;   // descriptor word 3: 32-bit data format, raw access
struct Span {
    __amdgpu_buffer_rsrc_t r;
    uint32_t end;   // bytes; an offset here stores nothing
    __device__ Span(const void* p, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, kBufWord3)), end(bytes) {}
    __device__ void st(bool ok, uint32_t byte_off, float v) const {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)(ok ? byte_off : end), 0, 0);
    }
    __device__ void st4(bool ok, uint32_t byte_off, const float* v) const {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 w = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)(ok ? byte_off : end), 0, 0);
    }
};

// Checkpoint record of (batch b, tile, channel d), tile-major: the records of
// consecutive channels at one tile are adjacent, so a block's checkpoint
// stores and loads of one tile cover one contiguous run (with the rows of a
// long sequence a power-of-two stride apart, a row-major layout sent every
// lane's store to its own far-apart line).
__device__ __forceinline__ int64_t ck_cell(const BwdArgs& a, int64_t b, int tile, int64_t d) {
    return (b * ((a.L + kT - 1) / kT) + tile) * a.dim + d;
}

struct Blk {
    int64_t b, cb, g, row0;       // row0 = b dim + 64 cb
    int t0, t_end, tiles, rows;   // rows: channels of this block below dim
    int L;                        // tokens
};

__device__ __forceinline__ Blk blk(const BwdArgs& a) {
    Blk k;
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    k.g = blockIdx.x % a.G;          // chunk fastest: neighbours share rows of B and C
    const int64_t rb = blockIdx.x / a.G;
    k.b = rb / nbc;
    k.cb = rb - k.b * nbc;
    k.row0 = k.b * a.dim + k.cb * kCh;
    k.L = (int)a.L;
    k.t0 = (int)(k.g * a.chunk);
    k.t_end = min(k.L, k.t0 + (int)a.chunk);
    k.tiles = (k.t_end - k.t0 + kT - 1) / kT;
    k.rows = (int)min<int64_t>(kCh, a.dim - k.cb * kCh);
    return k;
}

// Consumer view: this lane's channel and its 4 states.
struct Con {
    int l, w, rr, q, r, rc;   // rc: r clamped below the block's rows
    bool ok;                  // channel < dim
    float Al2[4];             // A[n] log2(e), 0 for padded states
    float A0l2;               // A[0] log2(e) of the channel
    bool st;                  // the lane's A[n] == fl32((n + 1) A[0]) and all 16 states real
    __device__ Con(const BwdArgs& a, const Blk& k) {
        const int tid = threadIdx.x;
        l = tid & 63;
        w = tid >> 6;
        rr = l & 3;
        q = (l >> 2) & 3;
        r = w * 16 + (l >> 4) * 4 + rr;
        ok = r < k.rows;
        rc = ok ? r : k.rows - 1;
        const float* Ab = a.A + k.cb * kCh * a.N;
        const float A0 = Ab[rc * a.N];
        A0l2 = A0 * kLog2e;
        st = a.N == kSt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 4 * q + i;
            const float An = n < a.N ? Ab[rc * a.N + n] : 0.0f;
            Al2[i] = An * kLog2e;
            st = st && An == (float)(n + 1) * A0;
        }
    }
};

// exp(Delta A[n]) of the lane's 4 states, dt = Delta.  With a structured A
// (A[n] = (n + 1) A[0] in every lane of the workgroup) they are consecutive
// powers r^(4q+1) .. r^(4q+4) of r = exp(Delta A[0]): two exponentials and
// three multiplies instead of four exponentials.
template <bool ST>
__device__ __forceinline__ void decay4(const Con& c, float dt, float at[4]) {
    if constexpr (ST) {
        const float r = fast_exp2(dt * c.A0l2);
        at[0] = fast_exp2(dt * c.Al2[0]);
        at[1] = at[0] * r;
        at[2] = at[1] * r;
        at[3] = at[2] * r;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) at[i] = fast_exp2(dt * c.Al2[i]);
    }
}

// True in every thread when every channel of the workgroup has a structured A
// (a workgroup-wide vote: all threads must call it).
__device__ __forceinline__ bool structured_block(const BwdArgs& a) {
    const Blk k = blk(a);
    const Con c(a, k);
    return __syncthreads_and(c.st ? 1 : 0) != 0;
}

// Producer view: channel pr, tokens pj .. pj + kPT - 1 of each tile.
struct Pro {
    int pr, pj, rc;
    bool ok;
    uint32_t off;   // rc * L: the channel's row within the block's rows
    float bias, D;
    __device__ Pro(const BwdArgs& a, const Blk& k) {
        const int tid = threadIdx.x;
        pr = tid >> 2;
        pj = (tid & 3) * kPT;
        ok = pr < k.rows;
        rc = ok ? pr : k.rows - 1;
        off = (uint32_t)rc * (uint32_t)k.L;
        const int64_t d = k.cb * kCh + rc;
        bias = a.bias ? a.bias[d] : 0.0f;
        D = a.D ? a.D[d] : 0.0f;
    }
};

// The block's rows of the per-token inputs, and its batch's B and C.
template <typename Tin, typename Tout>
struct In {
    const Tin *delta, *u, *z, *B, *C;
    const Tout* dout;
    __device__ In(const BwdArgs& a, const Blk& k) {
        const int64_t o = k.row0 * a.L;
        delta = reinterpret_cast<const Tin*>(a.delta) + o;
        u = reinterpret_cast<const Tin*>(a.u) + o;
        // without a gate: a valid address whose values are ignored
        z = reinterpret_cast<const Tin*>(a.z ? a.z : a.delta) + o;
        dout = reinterpret_cast<const Tout*>(a.dout) + o;
        B = reinterpret_cast<const Tin*>(a.B) + k.b * a.N * a.L;
        C = reinterpret_cast<const Tin*>(a.C) + k.b * a.N * a.L;
    }
};

// A producer thread's raw inputs for its kPT tokens of one tile, and one
// entry of the tile's B and C, loaded a tile ahead of their use.
// The loads are unconditional, from clamped in-bounds addresses, and the raw
// bits are kept: the loads stay in flight until the values are used, where
// tokens past the sequence and channels past dim are masked to zero.
template <typename Tin, typename Tout>
struct Raw {
    Tin x[kPT], u[kPT], z[kPT];
    Tout g[kPT];
    Tin bv, cv;
};

__device__ __forceinline__ float f32_of(float v) { return v; }
__device__ __forceinline__ float f32_of(uint16_t v) { return bf16_to_f32(v); }

// U: u, Z: z and dout, BB: B, CC: C.
template <typename Tin, typename Tout, bool U, bool Z, bool BB, bool CC>
__device__ __forceinline__ void fetch_raw(const BwdArgs& a, const Blk& k, const Pro& p, const In<Tin, Tout>& in,
                                          int tt0, Raw<Tin, Tout>& r) {
#pragma unroll
    for (int jj = 0; jj < kPT; ++jj) {
        const uint32_t o = p.off + (uint32_t)min(tt0 + p.pj + jj, k.L - 1);
        r.x[jj] = ldo(in.delta, o);
        if (U) r.u[jj] = ldo(in.u, o);
        if (Z) {
            r.g[jj] = ldo(in.dout, o);
            r.z[jj] = ldo(in.z, o);
        }
    }
    {   // thread (j, n) holds entry (j, n) (threads past kT x 16 load a duplicate)
        const int j = (threadIdx.x >> 4) & (kT - 1), n = min<int>(threadIdx.x & 15, a.N - 1);
        const uint32_t o = (uint32_t)n * (uint32_t)k.L + (uint32_t)min(tt0 + j, k.L - 1);
        if (BB) r.bv = ldo(in.B, o);
        if (CC) r.cv = ldo(in.C, o);
    }
}

// whether entry (j, n) of a B/C tile is a real value
__device__ __forceinline__ bool bc_valid(const BwdArgs& a, const Blk& k, int tt0) {
    const int j = threadIdx.x >> 4, n = threadIdx.x & 15;
    return n < a.N && tt0 + j < k.t_end;
}

// Tile values by tile parity: the producers fill one copy while the
// consumers may still read the other, so each tile needs one barrier.
struct SumSmem {
    float dt[2][kCh][kPad];
    float x2[2][kCh][kPad];  // Delta u (forward) or dy (reverse)
    alignas(16) float bc[2][kT][kSt];   // B (forward) or C (reverse); read as float4
};

// Per chunk, from zero: state every tile and at the end, running sum of
// Delta; and (when the sequence has several chunks) the adjoint leaving the
// chunk's first token, a_{t0} lam_{t0}, from a zero right boundary.
template <typename Tin, typename Tout, bool SP, bool ST>
__device__ __forceinline__ void summary_body(const BwdArgs& a, SumSmem& sm) {
    const Blk k = blk(a);
    const Con c(a, k);
    const Pro p(a, k);
    const In<Tin, Tout> in(a, k);
    const int tid = threadIdx.x;
    const int tile0 = k.t0 / kT;
    const bool bc_thread = tid < kT * kSt;
    const int bj = (tid >> 4) & (kT - 1), bn = tid & 15;

    float h[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float W = 0.0f;
    Raw<Tin, Tout> r;
    fetch_raw<Tin, Tout, true, false, true, false>(a, k, p, in, k.t0, r);
    for (int tile = 0; tile < k.tiles; ++tile) {
        const int tt0 = k.t0 + tile * kT;
        const int pb = tile & 1;
#pragma unroll
        for (int jj = 0; jj < kPT; ++jj) {
            float dd;
            const float dt = delta_of<SP>(f32_of(r.x[jj]) + p.bias, dd);
            const bool ok = p.ok && tt0 + p.pj + jj < k.t_end;
            sm.dt[pb][p.pr][p.pj + jj] = ok ? dt : 0.0f;
            sm.x2[pb][p.pr][p.pj + jj] = ok ? dt * f32_of(r.u[jj]) : 0.0f;
        }
        if (bc_thread) sm.bc[pb][bj][bn] = bc_valid(a, k, tt0) ? f32_of(r.bv) : 0.0f;
        {
            const int64_t ct = ck_cell(a, k.b, tile0 + tile, k.cb * kCh);
            Span(a.ckz + ct * kSt, (uint32_t)k.rows * (kSt * 4)).st4(c.ok, (uint32_t)(c.rc * 4 + c.q) * 16, h);
            Span(a.wck + ct, (uint32_t)k.rows * 4).st(c.ok && c.q == 0, (uint32_t)c.rc * 4, W);
        }
        lds_barrier();
        // unconditional (the last tile re-fetches itself): no branch around the loads
        fetch_raw<Tin, Tout, true, false, true, false>(a, k, p, in, k.t0 + min(tile + 1, k.tiles - 1) * kT, r);
        // keeps the loads here, a tile ahead of their use (the compiler
        // would otherwise sink them to the next tile, next to their use)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < kT; ++j) {
            const float dt = sm.dt[pb][c.r][j], dtu = sm.x2[pb][c.r][j];
            const float4 Bv = *reinterpret_cast<const float4*>(&sm.bc[pb][j][4 * c.q]);
            const float bb[4] = {Bv.x, Bv.y, Bv.z, Bv.w};
            W += dt;
            float at[4];
            decay4<ST>(c, dt, at);
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = __builtin_fmaf(at[i], h[i], dtu * bb[i]);
        }
        // no barrier: the next tile's values go to the other copy, and the
        // one after it is written only past the next tile's barrier, which
        // every thread reaches after reading this copy
    }
    const int G = (int)a.G;
    const uint32_t cg = (uint32_t)c.rc * (uint32_t)G + (uint32_t)k.g;
    const uint32_t cell = cg * kSt + 4 * c.q;
    float* hbuf = a.hbuf + k.row0 * G * kSt;
    if (c.ok) {
        *reinterpret_cast<float4*>(hbuf + cell) = make_float4(h[0], h[1], h[2], h[3]);
        if (c.q == 0) (a.wbuf + k.row0 * G)[cg] = W;
    }
    if (G == 1) return;   // uniform over the grid

    float mu[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    fetch_raw<Tin, Tout, false, true, false, true>(a, k, p, in, k.t0 + (k.tiles - 1) * kT, r);
    // every thread is past its reads of the forward sweep's last tile
    lds_barrier();
    for (int tile = k.tiles - 1; tile >= 0; --tile) {
        const int tt0 = k.t0 + tile * kT;
        const int pb = tile & 1;
#pragma unroll
        for (int jj = 0; jj < kPT; ++jj) {
            float dd;
            const float dt = delta_of<SP>(f32_of(r.x[jj]) + p.bias, dd);
            const bool ok = p.ok && tt0 + p.pj + jj < k.t_end;
            const float g = f32_of(r.g[jj]);
            float dy = g;
            if (a.z) {
                const float zz = f32_of(r.z[jj]);
                dy = g * zz * sigmoid(zz);
            }
            sm.dt[pb][p.pr][p.pj + jj] = ok ? dt : 0.0f;
            sm.x2[pb][p.pr][p.pj + jj] = ok ? dy : 0.0f;
        }
        if (bc_thread) sm.bc[pb][bj][bn] = bc_valid(a, k, tt0) ? f32_of(r.cv) : 0.0f;
        lds_barrier();
        fetch_raw<Tin, Tout, false, true, false, true>(a, k, p, in, k.t0 + max(tile - 1, 0) * kT, r);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = kT - 1; j >= 0; --j) {
            const float dt = sm.dt[pb][c.r][j], dy = sm.x2[pb][c.r][j];
            const float4 Cv = *reinterpret_cast<const float4*>(&sm.bc[pb][j][4 * c.q]);
            const float cc[4] = {Cv.x, Cv.y, Cv.z, Cv.w};
            float at[4];
            decay4<ST>(c, dt, at);
#pragma unroll
            for (int i = 0; i < 4; ++i) mu[i] = at[i] * __builtin_fmaf(dy, cc[i], mu[i]);
        }
    }
    if (c.ok) *reinterpret_cast<float4*>(a.mubuf + k.row0 * G * kSt + cell) = make_float4(mu[0], mu[1], mu[2], mu[3]);
}

template <typename Tin, typename Tout, bool SP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void m1_bwd_summary_kernel(BwdArgs a) {
    __shared__ SumSmem sm;
    if (structured_block(a))
        summary_body<Tin, Tout, SP, true>(a, sm);
    else
        summary_body<Tin, Tout, SP, false>(a, sm);
}

// ---------------------------------------------------------------------------
// The summary pass with one channel per lane, for rows of u, delta, z and
// dout that start on 16-byte boundaries: the same quantities as
// m1_bwd_summary_kernel (checkpoints every tile, the chunk's end state and
// sum of Delta, the adjoint leaving its first token), computed the way the
// forward scan runs: a wave covers 64 channels, a lane keeps its channel's 16
// states in registers, 32-token tiles of the rows arrive by row copies into
// LDS (lds_rows.hpp) and each token's B (forward sweep) or C (reverse sweep)
// record is read as a broadcast from the tile's copy of the fp32 records.
// No barriers and no cross-lane sums: the 4-lanes-per-channel layout is kept
// for the chunk pass, whose dB and dC are sums over channels.
namespace lane_summary {

constexpr int kTile = 32;   // tokens per row copy
constexpr int kBlk = 8;     // tokens per block read from LDS into registers
static_assert(kTile % kT == 0 && kT % kBlk == 0, "checkpoints fall on block starts");

// An 8-token block of one row: 4 words of bf16 or 8 of fp32.
template <typename T> struct Elt;
template <> struct Elt<float> {
    static constexpr int kW = 8;
    static __device__ __forceinline__ float get(const uint32_t* w, int j) { return __uint_as_float(w[j]); }
};
template <> struct Elt<uint16_t> {
    static constexpr int kW = 4;
    static __device__ __forceinline__ float get(const uint32_t* w, int j) {
        return (j & 1) ? bf16hi(w[j >> 1]) : bf16lo(w[j >> 1]);
    }
};

// Block blk of tensor t of an image (lds_rows.hpp layout) starting at uint4 `img`.
template <typename T>
__device__ __forceinline__ void read_block(uint32_t* w, const uint4* img, int t, int blk, int ls) {
    constexpr int per = Elt<T>::kW / 4;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        const uint4 x = img[rows::piece_slot<T>(t, blk * per + q, ls)];
        w[4 * q] = x.x; w[4 * q + 1] = x.y; w[4 * q + 2] = x.z; w[4 * q + 3] = x.w;
    }
}

// B (off 0) or C (off 16) halves of the records of tokens t .. t+31:
// 64 bytes per token, 16 tokens per instruction.
__device__ __forceinline__ void issue_half(const float* bcb, int t, uint32_t base, int off) {
    const int lane = threadIdx.x;
    const float* g = bcb + (int64_t)(t + (lane >> 2)) * (2 * kSt) + off + (lane & 3) * 4;
    rows::dma_at<0>(g, base);
    rows::dma_at<2048>(g, base + 1024);
}

// exp(Delta A[n]) for the 16 states, dt = Delta: powers of one exponential
// when A is structured (A[n] = (n+1) A[0]), else one exponential each.
template <bool ST>
__device__ __forceinline__ void decay16(const float* Al2, float dt, float* a) {
    if constexpr (ST) {
        const float r = fast_exp2(dt * Al2[0]);
        a[0] = r;
        a[1] = r * r;
        a[2] = a[1] * r;
        a[3] = a[1] * a[1];
#pragma unroll
        for (int n = 4; n < kSt; ++n) a[n] = a[n - 4] * a[3];
    } else {
#pragma unroll
        for (int n = 0; n < kSt; ++n) a[n] = fast_exp2(dt * Al2[n]);
    }
}

template <typename T>
__device__ __forceinline__ float ld1(const T* p, int i) { return f32_of(p[i]); }

// Ends a token: its 16 states are final here, and neither the next token's
// record reads nor its updates move above this point.  (Without it the
// compiler reads all of a block's records first and keeps them in registers,
// which spills.)
__device__ __forceinline__ void token_fence(float* v) {
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                 "+v"(v[7]), "+v"(v[8]), "+v"(v[9]), "+v"(v[10]), "+v"(v[11]), "+v"(v[12]), "+v"(v[13]),
                 "+v"(v[14]), "+v"(v[15])
                 :
                 : "memory");
}

// LDS of one wave: the rows' images (forward: u, delta; reverse: delta, z,
// then dout), then two buffers of 32 half-records.
template <typename Tin, typename Tout>
constexpr int kRowKB = 2 * rows::kPieces<Tin> + rows::kPieces<Tout>;

template <typename Tin, typename Tout, bool SP, bool ST>
__device__ __forceinline__ void body(const BwdArgs& a, uint4* lds) {
    const int lane = threadIdx.x;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(rows::ldsptr)lds;
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    const int G = (int)a.G;
    const int g = (int)(blockIdx.x % a.G);      // chunk fastest, as in the other passes
    const int64_t rb = blockIdx.x / a.G;
    const int64_t b = rb / nbc;
    const int64_t d0 = (rb - b * nbc) * kCh;
    const int last = (int)min<int64_t>(kCh, a.dim - d0) - 1;
    const bool row_ok = lane <= last;
    const int rc = min(lane, last);
    const int64_t row0 = b * a.dim + d0;
    const int L = (int)a.L;
    const int t0 = (int)(g * a.chunk);
    const int t_end = min(L, t0 + (int)a.chunk);
    const int t_full = t0 + ((t_end - t0) / kTile) * kTile;
    const int ls = rows::lane_slot(lane);

    float Al2[kSt];
#pragma unroll
    for (int n = 0; n < kSt; ++n) Al2[n] = n < a.N ? a.A[(d0 + rc) * a.N + n] * kLog2e : 0.0f;
    const float bias = a.bias ? a.bias[d0 + rc] : 0.0f;
    const float* bcb = rows::uniform(a.bcq + (int64_t)b * L * (2 * kSt));
    const uint32_t bc_base0 = lds_base + (uint32_t)kRowKB<Tin, Tout> * 1024u;
    const float* bcl0 = reinterpret_cast<const float*>(lds + kRowKB<Tin, Tout> * 64);
    const Tin* urow0 = reinterpret_cast<const Tin*>(a.u) + row0 * a.L;
    const Tin* drow0 = reinterpret_cast<const Tin*>(a.delta) + row0 * a.L;
    const Tin* zrow0 = a.z ? reinterpret_cast<const Tin*>(a.z) + row0 * a.L : drow0;
    const Tout* grow0 = reinterpret_cast<const Tout*>(a.dout) + row0 * a.L;
    const int64_t ro = (int64_t)rc * a.L;   // this lane's row within the block's rows

    float h[kSt];
#pragma unroll
    for (int n = 0; n < kSt; ++n) h[n] = 0.0f;
    float W = 0.0f;
    // checkpoints: the state entering tile t / kT and the sum of Delta before
    // it; the block's 64 records of one tile are contiguous
    auto ckpt = [&](int t) {
        const int64_t ct = ck_cell(a, b, t / kT, d0);
        const Span ckz(a.ckz + ct * kSt, (uint32_t)(last + 1) * (kSt * 4));
#pragma unroll
        for (int q = 0; q < kSt / 4; ++q) ckz.st4(row_ok, (uint32_t)(rc * kSt + 4 * q) * 4, &h[4 * q]);
        Span(a.wck + ct, (uint32_t)(last + 1) * 4).st(row_ok, (uint32_t)rc * 4, W);
    };
    auto fwd_token = [&](float dl, float uu, const float* Bp) {
        float dd;
        const float dt = delta_of<SP>(dl + bias, dd);
        const float x = dt * uu;
        float at[kSt];
        decay16<ST>(Al2, dt, at);
#pragma unroll
        for (int n = 0; n < kSt; ++n) h[n] = __builtin_fmaf(at[n], h[n], x * Bp[n]);
        W += dt;
        token_fence(h);
    };

    // forward sweep from a zero state
    rows::RowDma<Tin> Rf;
    Rf.init(urow0, drow0, drow0, a.L, last, lane);
    if (t0 < t_full) {
        rows::issue_rows<Tin, 2>(Rf, t0, lds_base);
        issue_half(bcb, t0, bc_base0, 0);
        rows::wait_vm();
        int par = 0;
#pragma nounroll
        for (int t = t0; t < t_full; t += kTile, par ^= 1) {
            const bool more = t + kTile < t_full;
            const float* bcl = bcl0 + par * (kTile * kSt);
            uint32_t cu[Elt<Tin>::kW], cd[Elt<Tin>::kW], nu[Elt<Tin>::kW], nd[Elt<Tin>::kW];
            read_block<Tin>(cu, lds, 0, 0, ls);
            read_block<Tin>(cd, lds, 1, 0, ls);
#pragma unroll
            for (int blk = 0; blk < kTile / kBlk; ++blk) {
                if (blk + 1 < kTile / kBlk) {
                    read_block<Tin>(nu, lds, 0, blk + 1, ls);
                    read_block<Tin>(nd, lds, 1, blk + 1, ls);
                }
                if (blk == kTile / kBlk - 2 && more) {
                    // the last two blocks are in registers and the other
                    // record buffer is free: request the next tile
                    rows::wait_lgkm();
                    rows::issue_rows<Tin, 2>(Rf, t + kTile, lds_base);
                    issue_half(bcb, t + kTile, bc_base0 + (uint32_t)((par ^ 1) * kTile * 64), 0);
                }
                if ((blk * kBlk) % kT == 0) ckpt(t + blk * kBlk);
#pragma unroll
                for (int j = 0; j < kBlk; ++j)
                    fwd_token(Elt<Tin>::get(cd, j), Elt<Tin>::get(cu, j), bcl + (blk * kBlk + j) * kSt);
                if (blk + 1 < kTile / kBlk) {
#pragma unroll
                    for (int i = 0; i < Elt<Tin>::kW; ++i) { cu[i] = nu[i]; cd[i] = nd[i]; }
                }
            }
            rows::wait_vm();
        }
    }
    // the rest of the chunk token by token
    for (int t = t_full; t < t_end; ++t) {
        if ((t - t0) % kT == 0) ckpt(t);
        fwd_token(ld1(drow0 + ro, t), ld1(urow0 + ro, t), bcb + (int64_t)t * (2 * kSt));
    }
    const uint32_t cell = ((uint32_t)rc * (uint32_t)G + (uint32_t)g) * kSt;
    float* hbuf = a.hbuf + row0 * G * kSt;
    if (row_ok) {
#pragma unroll
        for (int q = 0; q < kSt / 4; ++q)
            *reinterpret_cast<float4*>(hbuf + cell + 4 * q) = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
        (a.wbuf + row0 * G)[(uint32_t)rc * (uint32_t)G + (uint32_t)g] = W;
    }
    if (G == 1) return;   // uniform over the grid

    // reverse sweep of the adjoint from a zero right boundary
    float mu[kSt];
#pragma unroll
    for (int n = 0; n < kSt; ++n) mu[n] = 0.0f;
    auto rev_token = [&](float dl, float gg, float zz, const float* Cp) {
        float dd;
        const float dt = delta_of<SP>(dl + bias, dd);
        const float dy = a.z ? gg * zz * sigmoid(zz) : gg;
        float at[kSt];
        decay16<ST>(Al2, dt, at);
#pragma unroll
        for (int n = 0; n < kSt; ++n) mu[n] = at[n] * __builtin_fmaf(dy, Cp[n], mu[n]);
        token_fence(mu);
    };
    for (int t = t_end - 1; t >= t_full; --t)
        rev_token(ld1(drow0 + ro, t), ld1(grow0 + ro, t), ld1(zrow0 + ro, t), bcb + (int64_t)t * (2 * kSt) + kSt);
    if (t0 < t_full) {
        rows::RowDma<Tin> Rr;
        Rr.init(drow0, zrow0, drow0, a.L, last, lane);
        rows::RowDma<Tout> Rg;
        Rg.init(grow0, grow0, grow0, a.L, last, lane);
        const uint32_t g_base = lds_base + (uint32_t)(2 * rows::kPieces<Tin>) * 1024u;
        const uint4* gimg = lds + 2 * rows::kPieces<Tin> * 64;
        auto issue = [&](int t, uint32_t bc) {
            rows::issue_rows<Tin, 2>(Rr, t, lds_base);
            rows::issue_rows<Tout, 1>(Rg, t, g_base);
            issue_half(bcb, t, bc, kSt);
        };
        issue(t_full - kTile, bc_base0);
        rows::wait_vm();
        int par = 0;
#pragma nounroll
        for (int t = t_full - kTile; t >= t0; t -= kTile, par ^= 1) {
            const bool more = t > t0;
            const float* bcl = bcl0 + par * (kTile * kSt);
            uint32_t cd[Elt<Tin>::kW], cz[Elt<Tin>::kW], cg[Elt<Tout>::kW];
            uint32_t nd[Elt<Tin>::kW], nz[Elt<Tin>::kW], ng[Elt<Tout>::kW];
            constexpr int NB = kTile / kBlk;
            read_block<Tin>(cd, lds, 0, NB - 1, ls);
            read_block<Tin>(cz, lds, 1, NB - 1, ls);
            read_block<Tout>(cg, gimg, 0, NB - 1, ls);
#pragma unroll
            for (int bi = 0; bi < NB; ++bi) {
                const int blk = NB - 1 - bi;
                if (blk > 0) {
                    read_block<Tin>(nd, lds, 0, blk - 1, ls);
                    read_block<Tin>(nz, lds, 1, blk - 1, ls);
                    read_block<Tout>(ng, gimg, 0, blk - 1, ls);
                }
                if (bi == NB - 2 && more) {
                    rows::wait_lgkm();
                    issue(t - kTile, bc_base0 + (uint32_t)((par ^ 1) * kTile * 64));
                }
#pragma unroll
                for (int j = kBlk - 1; j >= 0; --j)
                    rev_token(Elt<Tin>::get(cd, j), Elt<Tout>::get(cg, j), Elt<Tin>::get(cz, j),
                              bcl + (blk * kBlk + j) * kSt);
                if (blk > 0) {
#pragma unroll
                    for (int i = 0; i < Elt<Tin>::kW; ++i) { cd[i] = nd[i]; cz[i] = nz[i]; }
#pragma unroll
                    for (int i = 0; i < Elt<Tout>::kW; ++i) cg[i] = ng[i];
                }
            }
            rows::wait_vm();
        }
    }
    if (row_ok) {
        float* mubuf = a.mubuf + row0 * G * kSt;
#pragma unroll
        for (int q = 0; q < kSt / 4; ++q)
            *reinterpret_cast<float4*>(mubuf + cell + 4 * q) =
                make_float4(mu[4 * q], mu[4 * q + 1], mu[4 * q + 2], mu[4 * q + 3]);
    }
}

// True when every state of channel d satisfies A[d,n] == fl32((n+1) A[d,0])
// and all 16 states are real.
__device__ __forceinline__ bool row_structured(const BwdArgs& a, int64_t d) {
    if (a.N != kSt) return false;
    const float A0 = a.A[d * a.N];
    bool s = true;
    for (int n = 1; n < a.N; ++n) s = s && (a.A[d * a.N + n] == (float)(n + 1) * A0);
    return s;
}

}  // namespace lane_summary

template <typename Tin, typename Tout, bool SP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void m1_bwd_lane_summary_kernel(BwdArgs a) {
    __shared__ uint4 lds[lane_summary::kRowKB<Tin, Tout> * 64 + 2 * lane_summary::kTile * kSt / 4];
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    const int64_t d0 = ((int64_t)(blockIdx.x / a.G) % nbc) * kCh;
    const int64_t d = min<int64_t>(d0 + threadIdx.x, a.dim - 1);
    const bool st = __builtin_amdgcn_ballot_w64(!lane_summary::row_structured(a, d)) == 0;
    if (st)
        lane_summary::body<Tin, Tout, SP, true>(a, lds);
    else
        lane_summary::body<Tin, Tout, SP, false>(a, lds);
}

// Per (row, n): the true state entering each chunk and the true adjoint
// entering it from the right, in place of the summaries.
__global__ __launch_bounds__(256) void m1_bwd_carry_kernel(BwdArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= a.batch * a.dim * kSt) return;
    const int64_t row = gid / kSt;
    const int n = (int)(gid - row * kSt);
    const int64_t d = row % a.dim;
    const float A = n < a.N ? a.A[d * a.N + n] * kLog2e : 0.0f;
    float* hb = a.hbuf + row * a.G * kSt + n;
    float* mb = a.mubuf + row * a.G * kSt + n;
    const float* wb = a.wbuf + row * a.G;
    float h = (a.h0 && n < a.N) ? a.h0[row * a.N + n] : 0.0f;
    for (int64_t g = 0; g < a.G; ++g) {
        const float loc = hb[g * kSt];
        hb[g * kSt] = h;
        h = __builtin_fmaf(fast_exp2(wb[g] * A), h, loc);
    }
    float mu = 0.0f;
    for (int64_t g = a.G - 1; g >= 0; --g) {
        const float loc = mb[g * kSt];
        mb[g * kSt] = mu;
        mu = __builtin_fmaf(fast_exp2(wb[g] * A), mu, loc);
    }
}

// Per-channel values of a tile, [channel][token] with the token index XORed
// by bits 1-2 of the channel.  Of 32 lanes the producer mapping touches 8
// channels at 4 consecutive tokens each, the adjoint lanes 8 channels at one
// token: with this layout either set falls in 32 distinct banks (a padded
// row pitch of 17 left the producer's accesses 2-way conflicted).
struct TileVals {
    float v[kCh * kT];
    __device__ __forceinline__ float& operator()(int r, int j) { return v[r * kT + (j ^ ((r >> 1) & 3))]; }
};

struct ChunkSmem {
    TileVals dt, dtu, dy;   // read by the adjoint lanes
    TileVals u, dd, zf;     // kept for the output pass
    alignas(16) float B[kT][kSt];   // read as float4
    alignas(16) float C[kT][kSt];
    TileVals sLB, sLAq, sCh;
    float red[kWaves][kT][2 * kSt];                       // per wave: dB[16], dC[16] per token
};

// One lane's 8 values (dB of states 4q..4q+3, then dC) summed over the wave's
// 16 channels (lane bits 0, 1: rr; bits 4, 5: the DPP row), scattered as
// they are summed: the half swap (bit 5) leaves dB in lanes 0..31 and dC in
// lanes 32..63, the row swap (bit 4) keeps states 4q + 2 b4 + {0, 1}, the
// quad exchange (bit 1) one of them, and bit 0 is summed last.  Returns kind
// b5 (0 = dB, 1 = dC) of state 4q + 2 b4 + b1, held by lanes l and l ^ 1.
// The swaps exchange values without a select per value: 16 instructions.
__device__ __forceinline__ float reduce_bc(const float* v, bool b1) {
    float u[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[m]), __float_as_uint(v[m + 4]), false, false);
        u[m] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
    float w[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[m]), __float_as_uint(u[m + 2]), false, false);
        w[m] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
    const float keep = b1 ? w[1] : w[0], send = b1 ? w[0] : w[1];
    const float x = keep + dpp<kQuadX2>(send);
    return x + dpp<kQuadX1>(x);
}

// Row images for the chunk pass (bf16 inputs, rows on 16-byte boundaries,
// chunks and L multiples of 32): 32 tokens of the block's rows of delta, u,
// z and dout copied into LDS 64 bytes per row per instruction
// (lds_rows.hpp), and the 32 tokens' fp32 B/C records.  Wave w copies row
// group w of every tensor and records 8w .. 8w+7.  An image serves two
// 16-token tiles; the producer mapping reads its 4 tokens per tensor from
// it instead of from global memory.
template <typename Tin, typename Tout>
struct ImgSmem {
    static constexpr int kIn = rows::kPieces<Tin>, kOut = rows::kPieces<Tout>;
    uint4 img[(3 * kIn + kOut) * 64];   // delta, u, z, then dout
    alignas(16) float rec[32][2 * kSt];
};

// This wave's row group of a 32-token image of one tensor (first row of the
// block at `row0`, `last` its last real row) into LDS at `slot0` (the
// tensor's image).
template <typename T>
__device__ __forceinline__ void img_rows(const T* row0, int64_t L, int last, int t, uint32_t slot0) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int k0 = min(16 * w, last);
    const char* g = reinterpret_cast<const char*>(row0 + (int64_t)(k0 + min(lane & 15, last - k0)) * L + t) +
                    16 * (lane >> 4);
    rows::dma_at<0>(g, slot0 + (uint32_t)w * 1024u);
    if constexpr (rows::kPieces<T> == 8) rows::dma_at<64>(g, slot0 + (uint32_t)(4 + w) * 1024u);
}

template <typename Tin, typename Tout, bool SP, bool ST, bool RI>
__device__ __forceinline__ void chunk_body(const BwdArgs& a, ChunkSmem& sm, ImgSmem<Tin, Tout>* im) {
    const Blk k = blk(a);
    const Con c(a, k);
    const Pro p(a, k);
    const In<Tin, Tout> in(a, k);
    const int tid = threadIdx.x;
    const int tile0 = k.t0 / kT;
    const int G = (int)a.G;
    const uint32_t cg = (uint32_t)c.rc * (uint32_t)G + (uint32_t)k.g;   // (channel, chunk) record
    const uint32_t cell = cg * kSt + 4 * c.q;
    const int64_t cell0 = k.row0 * G * kSt;
    const bool bc_thread = tid < kT * kSt;
    const int bj = (tid >> 4) & (kT - 1), bn = tid & 15;

    // state entering the chunk and adjoint entering it from the right
    // (c.rc is clamped in bounds: loads are unconditional, results masked)
    float h_in[4] = {0.0f, 0.0f, 0.0f, 0.0f}, lamn[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (G > 1) {
        const float4 hv = *reinterpret_cast<const float4*>(a.hbuf + cell0 + cell);
        const float4 mv = *reinterpret_cast<const float4*>(a.mubuf + cell0 + cell);
        h_in[0] = hv.x; h_in[1] = hv.y; h_in[2] = hv.z; h_in[3] = hv.w;
        lamn[0] = mv.x; lamn[1] = mv.y; lamn[2] = mv.z; lamn[3] = mv.w;
    } else if (a.h0) {
        const float* h0 = a.h0 + k.row0 * a.N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 4 * c.q + i;
            h_in[i] = h0[c.rc * a.N + min(n, a.N - 1)] * (n < a.N ? 1.0f : 0.0f);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h_in[i] = c.ok ? h_in[i] : 0.0f;
        lamn[i] = c.ok ? lamn[i] : 0.0f;
    }
    float dA[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float dD_acc = 0.0f, dbias_acc = 0.0f;
    // identity of this lane's dB/dC share
    const bool b1 = (c.l >> 1) & 1;
    const int vidx = (c.l >> 5) * kSt + 4 * c.q + 2 * ((c.l >> 4) & 1) + (int)b1;
    const bool writer = (c.l & 1) == 0;

    // prefetched inputs of the next tile (processed from the last)
    Raw<Tin, Tout> r;
    float4 zck;
    float wc;
    auto fetch = [&](int tile) {   // c.rc is clamped in bounds
        if constexpr (!RI) fetch_raw<Tin, Tout, true, true, true, true>(a, k, p, in, k.t0 + tile * kT, r);
        const int64_t ct = ck_cell(a, k.b, tile0 + tile, k.cb * kCh);
        zck = ldo(reinterpret_cast<const float4*>(a.ckz + ct * kSt), (uint32_t)c.rc * 4 + c.q);
        wc = ldo(a.wck + ct, (uint32_t)c.rc);
    };
    // image q covers tokens t0 + 32q .. t0 + 32q + 31 (tiles 2q, 2q + 1)
    const int img_last = (int)min<int64_t>(kCh, a.dim - k.cb * kCh) - 1;
    auto issue_img = [&](int q) {
        if constexpr (RI) {
            const int t = k.t0 + 32 * q;
            const uint32_t base = (uint32_t)(uintptr_t)(rows::ldsptr)im->img;
            constexpr int kIn = ImgSmem<Tin, Tout>::kIn;
            const int64_t o = k.row0 * a.L;
            img_rows<Tin>(reinterpret_cast<const Tin*>(a.delta) + o, a.L, img_last, t, base);
            img_rows<Tin>(reinterpret_cast<const Tin*>(a.u) + o, a.L, img_last, t, base + kIn * 1024u);
            img_rows<Tin>(reinterpret_cast<const Tin*>(a.z ? a.z : a.delta) + o, a.L, img_last, t,
                          base + 2 * kIn * 1024u);
            img_rows<Tout>(reinterpret_cast<const Tout*>(a.dout) + o, a.L, img_last, t, base + 3 * kIn * 1024u);
            const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
            const float* g = a.bcq + ((int64_t)k.b * a.L + t + 8 * w + (lane >> 3)) * (2 * kSt) + (lane & 7) * 4;
            rows::dma_at<0>(g, (uint32_t)(uintptr_t)(rows::ldsptr)&im->rec[0][0] + (uint32_t)w * 1024u);
        }
    };
    if constexpr (RI) issue_img(k.tiles / 2 - 1);
    fetch(k.tiles - 1);

    // the block's rows of du, ddelta, dz (at most 64 rows x 2^22 tokens x 4
    // bytes) and its dB/dC partials; no dz: an empty span, nothing stored
    const uint32_t row_bytes = (uint32_t)k.rows * (uint32_t)k.L * 4;
    const Span du(a.du + k.row0 * a.L, row_bytes);
    const Span ddelta(a.ddelta + k.row0 * a.L, row_bytes);
    const Span dz(a.dz ? a.dz + k.row0 * a.L : a.du, a.dz ? row_bytes : 0);
    const Span part(a.part + (k.cb * a.batch + k.b) * a.L * (2 * kSt), (uint32_t)k.L * (2 * kSt * 4));
    // Stores that store nothing, in the number each tile issues after its
    // prefetch: the first tile then finds the same memory operations in
    // flight as every later one (prefetch, then stores), and the compiler's
    // wait for the prefetch need not cover the previous tile's stores.
    // (With row images every tile is whole, and a producer thread's kPT
    // tokens, consecutive and 16-byte aligned, go out as one store per tensor.)
    constexpr int kGradSt = RI ? 1 : kPT;
#pragma unroll
    for (int jj = 0; jj < kGradSt; ++jj) {
        du.st(false, 0, 0.0f);
        ddelta.st(false, 0, 0.0f);
        dz.st(false, 0, 0.0f);
    }
#pragma unroll
    for (int jh = 0; jh < kT / kRT; ++jh) part.st(false, 0, 0.0f);
    for (int tile = k.tiles - 1; tile >= 0; --tile) {
        const int tt0 = k.t0 + tile * kT;
        float vx[kPT], vu[kPT], vz[kPT], vg[kPT], vb = 0.0f, vc = 0.0f;
        if constexpr (RI) {
            if (tile & 1) {   // first tile of an image: this wave's copies are in, then everyone's
                rows::wait_vm();
                lds_barrier();
            }
            // this thread's 4 tokens of row pr from the image's half tile & 1
            constexpr int kIn = ImgSmem<Tin, Tout>::kIn;
            const int pos = (tile & 1) * kT + p.pj;
            const int ls = rows::lane_slot(p.pr);
            auto four = [&](const uint4* base, int t, auto tag, float* v) {
                using T = decltype(tag);
                const char* q = reinterpret_cast<const char*>(base + rows::piece_slot<T>(t, pos * (int)sizeof(T) / 16, ls)) +
                                (pos * (int)sizeof(T)) % 16;
                if constexpr (sizeof(T) == 2) {
                    const uint2 w = *reinterpret_cast<const uint2*>(q);
                    v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
                } else {
                    const uint4 w = *reinterpret_cast<const uint4*>(q);
                    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
                    v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
                }
            };
            four(im->img, 0, Tin{}, vx);
            four(im->img, 1, Tin{}, vu);
            four(im->img, 2, Tin{}, vz);
            four(im->img + 3 * kIn * 64, 0, Tout{}, vg);
            vb = im->rec[(tile & 1) * kT + bj][bn];
            vc = im->rec[(tile & 1) * kT + bj][kSt + bn];
        } else {
#pragma unroll
            for (int jj = 0; jj < kPT; ++jj) {
                vx[jj] = f32_of(r.x[jj]); vu[jj] = f32_of(r.u[jj]);
                vz[jj] = f32_of(r.z[jj]); vg[jj] = f32_of(r.g[jj]);
            }
            vb = f32_of(r.bv);
            vc = f32_of(r.cv);
        }
        // per-channel tile values
#pragma unroll
        for (int jj = 0; jj < kPT; ++jj) {
            const int j = p.pj + jj;
            const bool ok = p.ok && tt0 + j < k.t_end;
            float dd;
            const float dt = delta_of<SP>(vx[jj] + p.bias, dd);
            const float g = vg[jj], uu = vu[jj];
            float dy = g, zf = 0.0f;
            if (a.z) {
                const float zz = vz[jj], sg = sigmoid(zz);
                dy = g * zz * sg;
                zf = g * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f);
            }
            sm.dt(p.pr, j) = ok ? dt : 0.0f;
            sm.dtu(p.pr, j) = ok ? dt * uu : 0.0f;
            sm.dy(p.pr, j) = ok ? dy : 0.0f;
            sm.u(p.pr, j) = uu;
            sm.dd(p.pr, j) = dd;
            sm.zf(p.pr, j) = zf;
        }
        if (bc_thread) {
            const bool ok = bc_valid(a, k, tt0);
            sm.B[bj][bn] = ok ? vb : 0.0f;
            sm.C[bj][bn] = ok ? vc : 0.0f;
        }
        lds_barrier();
        // every thread has read the image: the second tile of an image
        // requests the next (earlier) one
        if constexpr (RI) {
            if (!(tile & 1) && tile > 0) issue_img(tile / 2 - 1);
        }
        // the tile's first state: zero-start checkpoint + decayed entering
        // state (taken from the prefetch registers before they are reused)
        float ck[4];
        {
            const float zz[4] = {zck.x, zck.y, zck.z, zck.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ck[i] = c.ok ? __builtin_fmaf(fast_exp2(wc * c.Al2[i]), h_in[i], zz[i]) : 0.0f;
        }
        // ck is computed here, before the next loads: the prefetch registers
        // are then free for them and the loop carries no copies (whose waits
        // would drain the prefetch every tile)
        asm volatile("" ::"v"(ck[0]), "v"(ck[1]), "v"(ck[2]), "v"(ck[3]) : "memory");
        fetch(tile > 0 ? tile - 1 : 0);   // unconditional: no branch around the loads

        // recompute the tile's states
        // the tile's states and decays, kept for the adjoint sweep (the
        // decays are not computed twice: 64 registers, which the two waves
        // per SIMD leave free)
        float hs[kT][4], as[kT][4];
        {
            float h[4] = {ck[0], ck[1], ck[2], ck[3]};
#pragma unroll
            for (int j = 0; j < kT; ++j) {
                const float dt = sm.dt(c.r, j), dtu = sm.dtu(c.r, j);
                const float4 Bv = *reinterpret_cast<const float4*>(&sm.B[j][4 * c.q]);
                const float bb[4] = {Bv.x, Bv.y, Bv.z, Bv.w};
                decay4<ST>(c, dt, as[j]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h[i] = __builtin_fmaf(as[j][i], h[i], dtu * bb[i]);
                    hs[j][i] = h[i];
                }
            }
        }
        // adjoint back through the tile
#pragma unroll
        for (int j = kT - 1; j >= 0; --j) {
            const float dt = sm.dt(c.r, j), dtu = sm.dtu(c.r, j), dy = sm.dy(c.r, j);
            const float4 Bv = *reinterpret_cast<const float4*>(&sm.B[j][4 * c.q]);
            const float4 Cv = *reinterpret_cast<const float4*>(&sm.C[j][4 * c.q]);
            const float bb[4] = {Bv.x, Bv.y, Bv.z, Bv.w};
            const float cc[4] = {Cv.x, Cv.y, Cv.z, Cv.w};
            float sLB = 0.0f, sLAq = 0.0f, sCh = 0.0f;
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float hp = j > 0 ? hs[j - 1][i] : ck[i];
                const float at = as[j][i];
                const float lam = __builtin_fmaf(dy, cc[i], lamn[i]);
                const float tq = lam * at * hp;
                sLB = __builtin_fmaf(lam, bb[i], sLB);
                sLAq = __builtin_fmaf(c.Al2[i], tq, sLAq);   // log2(e) sum_n A lam a h_prev
                dA[i] = __builtin_fmaf(dt, tq, dA[i]);
                sCh = __builtin_fmaf(cc[i], hs[j][i], sCh);
                v[i] = lam * dtu;
                v[4 + i] = dy * hs[j][i];
                lamn[i] = at * lam;
            }
            sLB = sum_q(sLB);
            sLAq = sum_q(sLAq);
            sCh = sum_q(sCh);
            if (c.q == 0) {
                sm.sLB(c.r, j) = sLB;
                sm.sLAq(c.r, j) = sLAq;
                sm.sCh(c.r, j) = sCh;
            }
            const float s = reduce_bc(v, b1);
            if (writer) sm.red[c.w][j][vidx] = s;
        }
        lds_barrier();

        // per-channel outputs (producer mapping)
        float gu[kPT], gd[kPT], gz[kPT];
#pragma unroll
        for (int jj = 0; jj < kPT; ++jj) {
            const int j = p.pj + jj;
            const bool ok = p.ok && tt0 + j < k.t_end;
            const float sLB = sm.sLB(p.pr, j), sLAq = sm.sLAq(p.pr, j), sCh = sm.sCh(p.pr, j);
            const float dt = sm.dt(p.pr, j), dy = sm.dy(p.pr, j), uu = sm.u(p.pr, j);
            gu[jj] = __builtin_fmaf(dt, sLB, p.D * dy);
            gd[jj] = __builtin_fmaf(uu, sLB, sLAq * kLn2) * sm.dd(p.pr, j);
            gz[jj] = __builtin_fmaf(p.D, uu, sCh) * sm.zf(p.pr, j);
            dD_acc += ok ? dy * uu : 0.0f;
            dbias_acc += ok ? gd[jj] : 0.0f;
        }
        if constexpr (RI) {
            const uint32_t o = (p.off + (uint32_t)(tt0 + p.pj)) * 4;
            du.st4(p.ok, o, gu);
            ddelta.st4(p.ok, o, gd);
            dz.st4(p.ok, o, gz);
        } else {
#pragma unroll
            for (int jj = 0; jj < kPT; ++jj) {
                const int t = tt0 + p.pj + jj;
                const bool ok = p.ok && t < k.t_end;
                const uint32_t o = (p.off + (uint32_t)t) * 4;
                du.st(ok, o, gu[jj]);
                ddelta.st(ok, o, gd[jj]);
                dz.st(ok, o, gz[jj]);
            }
        }
#pragma unroll
        for (int jh = 0; jh < kT / kRT; ++jh) {   // dB, dC partials of this channel block: thread = (token j, value v)
            const int j = jh * kRT + (tid >> 5), v = tid & 31;
            const int t = tt0 + j;
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += sm.red[w][j][v];
            part.st(t < k.t_end, ((uint32_t)t * (2 * kSt) + v) * 4, s);
        }
        // No barrier needed before the next tile: a producer thread rewrites
        // only the entries it has just read itself, sm.B/C were last read
        // before the barrier above, and sm.sLB/sLAq/sCh/red are rewritten only
        // after the next tile's first barrier.
    }

    if (c.ok) {
        *reinterpret_cast<float4*>(a.pA + cell0 + cell) = make_float4(dA[0], dA[1], dA[2], dA[3]);
        if (k.g == 0 && a.dh0) {
            float* dh0 = a.dh0 + k.row0 * a.N;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 4 * c.q + i;
                if (n < a.N) dh0[c.rc * a.N + n] = lamn[i];   // a_0 lam_0
            }
        }
    }
    // dD, dbias: sum over the 4 producer threads of a channel (a quad)
    dD_acc += dpp<kQuadX1>(dD_acc);
    dD_acc += dpp<kQuadX2>(dD_acc);
    dbias_acc += dpp<kQuadX1>(dbias_acc);
    dbias_acc += dpp<kQuadX2>(dbias_acc);
    if (p.ok && (tid & 3) == 0) {
        const uint32_t pg = (uint32_t)p.rc * (uint32_t)G + (uint32_t)k.g;
        (a.pD + k.row0 * G)[pg] = dD_acc;
        (a.pbias + k.row0 * G)[pg] = dbias_acc;
    }
}

// 2 waves per SIMD: the tile's 16 recomputed states per lane need the
// registers (3 would spill).
template <typename Tin, typename Tout, bool SP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void m1_bwd_chunk_kernel(BwdArgs a) {
    __shared__ ChunkSmem sm;
    if (structured_block(a))
        chunk_body<Tin, Tout, SP, true, false>(a, sm, nullptr);
    else
        chunk_body<Tin, Tout, SP, false, false>(a, sm, nullptr);
}

// The chunk pass with row images (see ImgSmem).
template <typename Tin, typename Tout, bool SP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void m1_bwd_chunk_img_kernel(BwdArgs a) {
    __shared__ ChunkSmem sm;
    __shared__ ImgSmem<Tin, Tout> im;
    if (structured_block(a))
        chunk_body<Tin, Tout, SP, true, true>(a, sm, &im);
    else
        chunk_body<Tin, Tout, SP, false, true>(a, sm, &im);
}

// dB, dC: sums of the channel-block partials; thread = (token, value) of 8
// tokens of one batch, partials read 128 bytes per token.
__global__ __launch_bounds__(256) void m1_bwd_bc_reduce_kernel(BwdArgs a) {
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    const int64_t tblocks = (a.L + kRT - 1) / kRT;
    const int64_t b = blockIdx.x / tblocks;
    const int64_t t = (blockIdx.x - b * tblocks) * kRT + (threadIdx.x >> 5);
    const int v = threadIdx.x & 31, n = v & (kSt - 1);
    if (t >= a.L) return;
    const float* src = a.part + (b * a.L + t) * (2 * kSt) + v;
    const int64_t stride = a.batch * a.L * (2 * kSt);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
    int64_t cb = 0;
    for (; cb + 4 <= nbc; cb += 4) {
        s0 += src[(cb + 0) * stride];
        s1 += src[(cb + 1) * stride];
        s2 += src[(cb + 2) * stride];
        s3 += src[(cb + 3) * stride];
    }
    for (; cb < nbc; ++cb) s0 += src[cb * stride];
    const float s = (s0 + s1) + (s2 + s3);
    if (n < a.N) (v < kSt ? a.dB : a.dC)[(b * a.N + n) * a.L + t] = s;
}

// dA, dD, dbias: one wave per channel sums the (batch, chunk) partials, each
// lane a fixed strided share, then a fixed butterfly over the wave.
__global__ __launch_bounds__(256) void m1_bwd_param_reduce_kernel(BwdArgs a) {
    const int64_t d = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    if (d >= a.dim) return;   // uniform per wave
    float acc[kSt + 2];
#pragma unroll
    for (int i = 0; i < kSt + 2; ++i) acc[i] = 0.0f;
    const int64_t recs = a.batch * a.G;
    for (int64_t e = l; e < recs; e += 64) {
        const int64_t b = e / a.G, g = e - b * a.G;
        const int64_t rg = (b * a.dim + d) * a.G + g;
        const float4* q = reinterpret_cast<const float4*>(a.pA + rg * kSt);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 x = q[m];
            acc[4 * m] += x.x; acc[4 * m + 1] += x.y; acc[4 * m + 2] += x.z; acc[4 * m + 3] += x.w;
        }
        acc[kSt] += a.pD[rg];
        acc[kSt + 1] += a.pbias[rg];
    }
#pragma unroll
    for (int i = 0; i < kSt + 2; ++i)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) acc[i] += __shfl_xor(acc[i], o, 64);
    if (l == 0) {
        for (int n = 0; n < a.N; ++n) a.dA[d * a.N + n] = acc[n];
        if (a.dD) a.dD[d] = acc[kSt];
        if (a.dbias) a.dbias[d] = acc[kSt + 1];
    }
}

hipError_t launch_reduces(const BwdArgs& a, hipStream_t stream);

template <typename Tin, typename Tout, bool SP>
hipError_t launch_sp(const BwdArgs& a, hipStream_t stream) {
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    const unsigned blocks = (unsigned)(a.batch * nbc * a.G);
    if (a.lane_sum) {
        {
            KTime kt("m1_bwd_bc_convert", stream);
            const hipError_t e = launch_m1_bc(a.B, a.C, a.batch, a.N, a.L, a.bcq, sizeof(Tin) == 2, stream);
            if (e != hipSuccess) return e;
        }
        KTime kt("m1_bwd_summary", stream);
        hipLaunchKernelGGL((m1_bwd_lane_summary_kernel<Tin, Tout, SP>), dim3(blocks), dim3(64), 0, stream, a);
    } else {
        KTime kt("m1_bwd_summary", stream);
        hipLaunchKernelGGL((m1_bwd_summary_kernel<Tin, Tout, SP>), dim3(blocks), dim3(kThreads), 0, stream, a);
    }
    if (a.G > 1) {
        KTime kt("m1_bwd_carry", stream);
        const int64_t cells = a.batch * a.dim * kSt;
        hipLaunchKernelGGL(m1_bwd_carry_kernel, dim3((unsigned)((cells + 255) / 256)), dim3(256), 0, stream, a);
    }
    {
        KTime kt("m1_bwd_chunk", stream);
        bool img = false;
        if constexpr (sizeof(Tin) == 2) {
            if (a.chunk_img) {
                hipLaunchKernelGGL((m1_bwd_chunk_img_kernel<Tin, Tout, SP>), dim3(blocks), dim3(kThreads), 0, stream, a);
                img = true;
            }
        }
        if (!img)
            hipLaunchKernelGGL((m1_bwd_chunk_kernel<Tin, Tout, SP>), dim3(blocks), dim3(kThreads), 0, stream, a);
    }
    return launch_reduces(a, stream);
}

hipError_t launch_reduces(const BwdArgs& a, hipStream_t stream) {
    {
        KTime kt("m1_bwd_bc_reduce", stream);
        const unsigned rb = (unsigned)(a.batch * ((a.L + kRT - 1) / kRT));
        hipLaunchKernelGGL(m1_bwd_bc_reduce_kernel, dim3(rb), dim3(256), 0, stream, a);
    }
    KTime kt("m1_bwd_param_reduce", stream);
    hipLaunchKernelGGL(m1_bwd_param_reduce_kernel, dim3((unsigned)((a.dim + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_dt(const BwdArgs& a, hipStream_t stream) {
    return a.softplus ? launch_sp<Tin, Tout, true>(a, stream) : launch_sp<Tin, Tout, false>(a, stream);
}

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int m1_bwd_tile() { return kT; }
int m1_bwd_max_chunk() { return 4096; }
int m1_bwd_channels_per_block() { return kCh; }

size_t m1_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t L, int64_t G) {
    const int64_t nbc = (dim + kCh - 1) / kCh;
    const size_t rows = (size_t)batch * dim;
    const size_t cells = rows * G;
    const size_t TL = (size_t)((L + kT - 1) / kT);
    return 3 * a256(cells * kSt * 4) + 3 * a256(cells * 4) + a256((size_t)nbc * batch * 2 * kSt * L * 4) +
           a256(rows * TL * kSt * 4) + a256(rows * TL * 4) + a256((size_t)batch * L * 2 * kSt * 4);
}

void m1_bwd_carve(BwdArgs& a, void* ws) {
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    const size_t rows = (size_t)a.batch * a.dim;
    const size_t cells = rows * a.G;
    const size_t TL = (size_t)((a.L + kT - 1) / kT);
    char* q = static_cast<char*>(ws);
    auto take = [&q](size_t bytes) {
        float* r = reinterpret_cast<float*>(q);
        q += a256(bytes);
        return r;
    };
    a.hbuf = take(cells * kSt * 4);
    a.mubuf = take(cells * kSt * 4);
    a.pA = take(cells * kSt * 4);
    a.wbuf = take(cells * 4);
    a.pD = take(cells * 4);
    a.pbias = take(cells * 4);
    a.part = take((size_t)nbc * a.batch * 2 * kSt * a.L * 4);
    a.ckz = take(rows * TL * kSt * 4);
    a.wck = take(rows * TL * 4);
    a.bcq = take((size_t)a.batch * a.L * 2 * kSt * 4);
}

hipError_t launch_m1_bwd(const BwdArgs& a, int in_bf16, int out_bf16, hipStream_t stream) {
    if (in_bf16 && out_bf16) return launch_dt<uint16_t, uint16_t>(a, stream);
    if (in_bf16) return launch_dt<uint16_t, float>(a, stream);
    if (out_bf16) return launch_dt<float, uint16_t>(a, stream);
    return launch_dt<float, float>(a, stream);
}

}  // namespace selscan
