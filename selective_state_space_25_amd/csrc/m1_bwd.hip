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
//   du_t     = dy_t D + sum_n lam_t[n] Delta_t B_t[n]
//   dDelta_t = sum_n lam_t[n] (B_t[n] u_t + A[n] a_t[n] h_{t-1}[n])
//   dA[n]    = sum_{b,t} lam_t[n] Delta_t a_t[n] h_{t-1}[n]
//
// Time is cut into chunks so that the grid fills the chip:
//   summary: per chunk, the state at its end from a zero start and the
//            adjoint leaving its first token from a zero right boundary;
//   carry:   the true state entering each chunk (forward over chunks, from
//            h0) and the true adjoint entering it from the right (backward
//            over chunks) -- both linear, so the chunk's decay exp(A sum Delta)
//            is all that links neighbours;
//   chunk:   per chunk, a forward sweep storing the state every 32 tokens in
//            LDS, then tiles from the last: recompute the tile's 32 states in
//            registers and run the adjoint back through them;
//   reduce:  the sums over channel blocks, batches and chunks.
// A workgroup is 1024 threads, one per (channel, state n) of 64 channels.
// Sums over n use shuffles in the 16-lane group of a channel; dB and dC, sums
// over channels, go over the wave's 4 channels by shuffles, over the 16
// waves through LDS, and over channel blocks in the reduce pass from
// per-block partials (no atomics: results do not depend on scheduling).
#include "device_math.hpp"
#include "kernels.hpp"

namespace selscan {

namespace {

constexpr int kCh = 64;        // channels per workgroup
constexpr int kSt = 16;        // states per channel (padded)
constexpr int kTile = 32;      // tokens per recomputed tile
constexpr int kMaxTiles = 16;  // tiles per chunk (checkpoints held in LDS)
constexpr int kThreads = kCh * kSt;
constexpr int kWaves = kThreads / 64;

template <typename T> __device__ __forceinline__ float ld1(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld1<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

__device__ __forceinline__ float sum16(float v) {
#pragma unroll
    for (int o = 1; o < kSt; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float sigmoid(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }

// One thread's (channel, state) view of the inputs.
template <typename Tin, typename Tout, bool SP>
struct Cell {
    const Tin *u, *dl, *z, *bn, *cn;
    const Tout* dout;
    float A;       // A[d, n] log2(e)
    float An;      // A[d, n]
    float D, bias;
    bool st_ok;    // n < N

    __device__ Cell(const BwdArgs& a, int64_t b, int64_t d, int n) {
        const int64_t row = b * a.dim + d;
        const int nn = n < a.N ? n : 0;
        st_ok = n < a.N;
        u = reinterpret_cast<const Tin*>(a.u) + row * a.L;
        dl = reinterpret_cast<const Tin*>(a.delta) + row * a.L;
        z = a.z ? reinterpret_cast<const Tin*>(a.z) + row * a.L : nullptr;
        bn = reinterpret_cast<const Tin*>(a.B) + (b * a.N + nn) * a.L;
        cn = reinterpret_cast<const Tin*>(a.C) + (b * a.N + nn) * a.L;
        dout = reinterpret_cast<const Tout*>(a.dout) + row * a.L;
        An = st_ok ? a.A[d * a.N + n] : 0.0f;
        A = An * kLog2e;
        D = a.D ? a.D[d] : 0.0f;
        bias = a.bias ? a.bias[d] : 0.0f;
    }
    // Delta_t (natural units) and dDelta/d(delta_t)
    __device__ __forceinline__ float dt(int64_t t, float& deriv) const {
        const float x = ld1(dl, t) + bias;
        if (SP) {
            deriv = sigmoid(x);
            return softplus_log2(x * kLog2e) * kLn2;
        }
        deriv = 1.0f;
        return x;
    }
    __device__ __forceinline__ float dt(int64_t t) const {
        float dd;
        return dt(t, dd);
    }
    __device__ __forceinline__ float bval(int64_t t) const { return st_ok ? ld1(bn, t) : 0.0f; }
    __device__ __forceinline__ float cval(int64_t t) const { return st_ok ? ld1(cn, t) : 0.0f; }
    // dL/dy_t = dout_t silu(z_t)
    __device__ __forceinline__ float dy(int64_t t) const {
        const float g = ld1(dout, t);
        if (!z) return g;
        const float zz = ld1(z, t);
        return g * zz * sigmoid(zz);
    }
    // h_t from h_{t-1}; w accumulates Delta
    __device__ __forceinline__ float advance(float h, int64_t t, float& w) const {
        const float d = dt(t);
        w += d;
        return __builtin_fmaf(fast_exp2(d * A), h, d * bval(t) * ld1(u, t));
    }
};

struct Place {
    int tid, wave, n, ch;
    int64_t b, cb, d, row, g, t0, len;
    bool ch_ok;
};

__device__ __forceinline__ Place place(const BwdArgs& a) {
    Place p;
    p.tid = threadIdx.x;
    p.wave = p.tid >> 6;
    p.n = p.tid & (kSt - 1);
    p.ch = p.tid >> 4;
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    // chunk fastest: neighbouring workgroups share rows of B and C
    p.g = blockIdx.x % a.G;
    const int64_t rb = blockIdx.x / a.G;
    p.b = rb / nbc;
    p.cb = rb - p.b * nbc;
    const int64_t d_raw = p.cb * kCh + p.ch;
    p.ch_ok = d_raw < a.dim;
    p.d = p.ch_ok ? d_raw : a.dim - 1;
    p.row = p.b * a.dim + p.d;
    p.t0 = p.g * a.chunk;
    p.len = min<int64_t>(a.chunk, a.L - p.t0);
    return p;
}

// Per chunk: state at the end from a zero start, sum of Delta, and the adjoint
// leaving the first token (a_{t0} lam_{t0}) from a zero right boundary.
template <typename Tin, typename Tout, bool SP>
__global__ __launch_bounds__(kThreads) void m1_bwd_summary_kernel(BwdArgs a) {
    const Place p = place(a);
    const Cell<Tin, Tout, SP> c(a, p.b, p.d, p.n);
    float h = 0.0f, w = 0.0f;
    for (int64_t s = 0; s < p.len; s += kTile) {
        const int cnt = (int)min<int64_t>(kTile, p.len - s);
        if (cnt == kTile) {
#pragma unroll
            for (int j = 0; j < kTile; ++j) h = c.advance(h, p.t0 + s + j, w);
        } else {
            for (int j = 0; j < cnt; ++j) h = c.advance(h, p.t0 + s + j, w);
        }
    }
    float mu = 0.0f;
    for (int64_t s = p.len; s > 0; s -= kTile) {
        const int cnt = (int)min<int64_t>(kTile, s);
        for (int j = 1; j <= cnt; ++j) {
            const int64_t t = p.t0 + s - j;
            const float lam = __builtin_fmaf(c.dy(t), c.cval(t), mu);
            mu = fast_exp2(c.dt(t) * c.A) * lam;
        }
    }
    if (p.ch_ok) {
        const int64_t cell = (p.row * a.G + p.g) * kSt + p.n;
        a.hbuf[cell] = h;
        a.mubuf[cell] = mu;
        if (p.n == 0) a.wbuf[p.row * a.G + p.g] = w;
    }
}

// Per (row, n): the true state entering each chunk and the true adjoint
// entering it from the right, in place of the summaries; dh0 = the adjoint
// leaving the first chunk.
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

struct ChunkSmem {
    float ck[kMaxTiles][kThreads];            // state before each tile
    float red[kWaves][kTile][2 * kSt + 1];    // per wave and token: dB[16], dC[16]
    float go[3][kCh][kTile + 1];              // per channel and token: du, ddelta, dz
};

template <typename Tin, typename Tout, bool SP>
__global__ __launch_bounds__(kThreads) void m1_bwd_chunk_kernel(BwdArgs a) {
    __shared__ ChunkSmem sm;
    const Place p = place(a);
    const Cell<Tin, Tout, SP> c(a, p.b, p.d, p.n);
    const int tiles = (int)((p.len + kTile - 1) / kTile);
    const int64_t cell = (p.row * a.G + p.g) * kSt + p.n;
    const float h_in = (a.h0 && p.n < a.N) ? a.h0[p.row * a.N + p.n] : 0.0f;

    {   // forward: the state before each tile
        float h = a.G > 1 ? a.hbuf[cell] : h_in;
        float w = 0.0f;
        for (int tl = 0; tl < tiles; ++tl) {
            sm.ck[tl][p.tid] = h;
            if (tl + 1 < tiles) {
#pragma unroll
                for (int j = 0; j < kTile; ++j) h = c.advance(h, p.t0 + tl * kTile + j, w);
            }
        }
    }

    float lam_next = a.G > 1 ? a.mubuf[cell] : 0.0f;   // a_{t+1} lam_{t+1} past the chunk's end
    float dA_acc = 0.0f, dD_acc = 0.0f, dbias_acc = 0.0f;
    for (int tl = tiles - 1; tl >= 0; --tl) {
        const int64_t t0 = p.t0 + tl * kTile;
        const int cnt = (int)min<int64_t>(kTile, p.len - tl * kTile);
        const float hprev = sm.ck[tl][p.tid];
        float hs[kTile];
        {
            float h = hprev, w = 0.0f;
#pragma unroll
            for (int j = 0; j < kTile; ++j) {
                if (j < cnt) h = c.advance(h, t0 + j, w);
                hs[j] = h;
            }
        }
#pragma unroll
        for (int j = kTile - 1; j >= 0; --j) {
            float cB = 0.0f, cC = 0.0f;
            if (j < cnt) {
                const int64_t t = t0 + j;
                const float uu = ld1(c.u, t);
                float dd;
                const float dt = c.dt(t, dd);
                const float bv = c.bval(t);
                const float cv = c.cval(t);
                const float h = hs[j];
                const float hp = j > 0 ? hs[j - 1] : hprev;
                const float g = ld1(c.dout, t);
                float dy = g, dz = 0.0f;
                if (c.z) {
                    const float zz = ld1(c.z, t);
                    const float sg = sigmoid(zz);
                    const float y = __builtin_fmaf(c.D, uu, sum16(cv * h));
                    dy = g * zz * sg;
                    dz = g * y * sg * __builtin_fmaf(zz, 1.0f - sg, 1.0f);
                }
                const float lam = __builtin_fmaf(dy, cv, lam_next);
                const float at = fast_exp2(dt * c.A);
                cC = dy * h;
                cB = lam * dt * uu;
                const float du = __builtin_fmaf(dy, c.D, sum16(lam * dt * bv));
                const float ddt = sum16(lam * __builtin_fmaf(c.An * at, hp, bv * uu));
                dA_acc = __builtin_fmaf(lam * dt * at, hp, dA_acc);
                lam_next = at * lam;
                const float dx = ddt * dd;
                if (p.n == 0) {
                    dD_acc = __builtin_fmaf(dy, uu, dD_acc);
                    dbias_acc += dx;
                    sm.go[0][p.ch][j] = du;
                    sm.go[1][p.ch][j] = dx;
                    sm.go[2][p.ch][j] = dz;
                }
            }
            if (!p.ch_ok) cB = cC = 0.0f;
            // sum over the wave's 4 channels (lanes 16 apart)
            cB += __shfl_xor(cB, 16, 64);
            cB += __shfl_xor(cB, 32, 64);
            cC += __shfl_xor(cC, 16, 64);
            cC += __shfl_xor(cC, 32, 64);
            if ((p.tid & 63) < kSt) {
                sm.red[p.wave][j][p.n] = cB;
                sm.red[p.wave][j][kSt + p.n] = cC;
            }
        }
        __syncthreads();
        {   // dB, dC partials of this channel block: thread = (value v, token j)
            const int v = p.tid >> 5, j = p.tid & 31;
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += sm.red[w][j][v];
            if (j < cnt) a.part[((p.cb * a.batch + p.b) * 2 * kSt + v) * a.L + t0 + j] = s;
        }
        {   // du, ddelta, dz: thread = (channel, token j), 32 channels at a time
            const int j = p.tid & 31;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int ch = half * 32 + (p.tid >> 5);
                const int64_t d = p.cb * kCh + ch;
                if (j < cnt && d < a.dim) {
                    const int64_t o = (p.b * a.dim + d) * a.L + t0 + j;
                    a.du[o] = sm.go[0][ch][j];
                    a.ddelta[o] = sm.go[1][ch][j];
                    if (c.z) a.dz[o] = sm.go[2][ch][j];
                }
            }
        }
        __syncthreads();
    }
    if (p.ch_ok) {
        a.pA[cell] = dA_acc;   // zero for padded states
        if (p.n == 0) {
            a.pD[p.row * a.G + p.g] = dD_acc;
            a.pbias[p.row * a.G + p.g] = dbias_acc;
        }
        // the adjoint of h0 leaves the first chunk
        if (p.g == 0 && a.dh0 && p.n < a.N) a.dh0[p.row * a.N + p.n] = lam_next;
    }
}

// dB, dC: sums of the channel-block partials; dA, dD, dbias: sums over
// batches and chunks.
__global__ __launch_bounds__(256) void m1_bwd_reduce_kernel(BwdArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    const int64_t tot_bc = a.batch * a.N * a.L;
    if (gid < tot_bc) {
        const int64_t t = gid % a.L;
        const int64_t bn = gid / a.L;
        const int64_t n = bn % a.N;
        const int64_t b = bn / a.N;
        float sb = 0.0f, sc = 0.0f;
        for (int64_t cb = 0; cb < nbc; ++cb) {
            const float* q = a.part + ((cb * a.batch + b) * 2 * kSt + n) * a.L + t;
            sb += q[0];
            sc += q[kSt * a.L];
        }
        a.dB[gid] = sb;
        a.dC[gid] = sc;
        return;
    }
    const int64_t i = gid - tot_bc;
    if (i < a.dim * a.N) {
        const int64_t d = i / a.N, n = i - d * a.N;
        float s = 0.0f;
        for (int64_t b = 0; b < a.batch; ++b)
            for (int64_t g = 0; g < a.G; ++g) s += a.pA[((b * a.dim + d) * a.G + g) * kSt + n];
        a.dA[i] = s;
        return;
    }
    const int64_t d = i - a.dim * a.N;
    if (d < a.dim) {
        float sd = 0.0f, sbias = 0.0f;
        for (int64_t b = 0; b < a.batch; ++b)
            for (int64_t g = 0; g < a.G; ++g) {
                sd += a.pD[(b * a.dim + d) * a.G + g];
                sbias += a.pbias[(b * a.dim + d) * a.G + g];
            }
        if (a.dD) a.dD[d] = sd;
        if (a.dbias) a.dbias[d] = sbias;
    }
}

template <typename Tin, typename Tout, bool SP>
hipError_t launch_sp(const BwdArgs& a, hipStream_t stream) {
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    const unsigned blocks = (unsigned)(a.batch * nbc * a.G);
    if (a.G > 1) {
        {
            KTime kt("m1_bwd_summary", stream);
            hipLaunchKernelGGL((m1_bwd_summary_kernel<Tin, Tout, SP>), dim3(blocks), dim3(kThreads), 0, stream, a);
        }
        KTime kt("m1_bwd_carry", stream);
        const int64_t cells = a.batch * a.dim * kSt;
        hipLaunchKernelGGL(m1_bwd_carry_kernel, dim3((unsigned)((cells + 255) / 256)), dim3(256), 0, stream, a);
    }
    {
        KTime kt("m1_bwd_chunk", stream);
        hipLaunchKernelGGL((m1_bwd_chunk_kernel<Tin, Tout, SP>), dim3(blocks), dim3(kThreads), 0, stream, a);
    }
    const int64_t total = a.batch * a.N * a.L + a.dim * a.N + a.dim;
    KTime kt("m1_bwd_reduce", stream);
    hipLaunchKernelGGL(m1_bwd_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_dt(const BwdArgs& a, hipStream_t stream) {
    return a.softplus ? launch_sp<Tin, Tout, true>(a, stream) : launch_sp<Tin, Tout, false>(a, stream);
}

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int m1_bwd_tile() { return kTile; }
int m1_bwd_max_chunk() { return kTile * kMaxTiles; }
int m1_bwd_channels_per_block() { return kCh; }

size_t m1_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t L, int64_t G) {
    const int64_t nbc = (dim + kCh - 1) / kCh;
    const size_t cells = (size_t)batch * dim * G;
    return 3 * a256(cells * kSt * 4) + 3 * a256(cells * 4) + a256((size_t)nbc * batch * 2 * kSt * L * 4);
}

void m1_bwd_carve(BwdArgs& a, void* ws) {
    const int64_t nbc = (a.dim + kCh - 1) / kCh;
    const size_t cells = (size_t)a.batch * a.dim * a.G;
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
}

hipError_t launch_m1_bwd(const BwdArgs& a, int in_bf16, int out_bf16, hipStream_t stream) {
    if (in_bf16 && out_bf16) return launch_dt<uint16_t, uint16_t>(a, stream);
    if (in_bf16) return launch_dt<uint16_t, float>(a, stream);
    if (out_bf16) return launch_dt<float, uint16_t>(a, stream);
    return launch_dt<float, float>(a, stream);
}

}  // namespace selscan
