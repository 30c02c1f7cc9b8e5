// kernels.hpp -- argument blocks and launchers shared by the host entry
// points and the HIP kernels (internal to libselscan; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "selscan.h"

namespace selscan {

// Records `msg` as the calling thread's selscan_last_error() and returns s.
selscan_status_t set_error(selscan_status_t s, const std::string& msg);

// Per-kernel timing bracket (no-op unless selscan_timing_enable(1)).
void ktime_mark(const char* kernel, hipStream_t stream, bool begin);
struct KTime {
    const char* name;
    hipStream_t stream;
    KTime(const char* n, hipStream_t s) : name(n), stream(s) { ktime_mark(name, stream, true); }
    ~KTime() { ktime_mark(name, stream, false); }
};

// Mamba-1.  Tensors as in selscan.h; ws_* point into the workspace.
struct M1Args {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* bias;
    void* y;
    float* last;
    const float* h0;  // [batch, dim, N] initial state, or NULL for zero
    float* ws_state;  // [rows, G, 16] chunk end states from a zero start
    float* ws_w;      // [rows, G] chunk sums of Delta / ln2
    float* bcq;       // [batch, L, 32] fp32 copy of B and C (B0..B15, C0..C15 per token)
    int64_t batch, dim, L;
    int64_t chunk;    // longest chunk in tokens; the kernels split a row's tiles evenly over G chunks
    int N;            // d_state
    int G;            // chunks per row
    int softplus;
    int vec_ok;       // rows of u, delta, z, y start on 16-byte boundaries (tile path)
    int force_general;
    int xcd_chunks;   // G is a multiple of 8 and chunk g runs on XCD g % 8 (1-D grid)
    int carry_scan;   // the carries come from a scan over the chunk summaries (its own
                      // kernel) rather than from a fold at the start of each chunk
};

int m1_padded_states(int N);
int m1_chunk_align(int in_bf16);
int m1_resident_waves_per_cu(int in_bf16);
int m1_rows_per_block();
int m1_waves_per_block();
size_t m1_bc_bytes(int64_t batch, int64_t L);
hipError_t launch_m1(const M1Args& a, int in_bf16, int out_bf16, hipStream_t stream);
// B, C [batch, N, L] -> bcq [batch, L, 32] fp32 records (zeros past N).
hipError_t launch_m1_bc(const void* B, const void* C, int64_t batch, int N, int64_t L, float* bcq, int in_bf16,
                        hipStream_t stream);

// Mamba-1 backward.  Inputs as for M1Args plus dout [batch, dim, L]
// (out dtype); gradients fp32 in the layouts of their inputs.  hbuf .. part
// point into the workspace (m1_bwd_carve).
struct BwdArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* bias;
    const float* h0;
    const void* dout;
    float *du, *ddelta, *dA, *dB, *dC, *dD, *dz, *dbias, *dh0;
    float* hbuf;    // [rows, G, 16] chunk-end states from zero, then states entering each chunk
    float* mubuf;   // [rows, G, 16] adjoint leaving each chunk from zero, then the one entering it
    float* wbuf;    // [rows, G] chunk sums of Delta
    float* pA;      // [rows, G, 16] per-chunk dA terms
    float* pD;      // [rows, G]
    float* pbias;   // [rows, G]
    float* part;    // [dim / 64, batch, L, 32] per-channel-block dB (16) and dC (16)
    float* ckz;     // [batch, tiles, dim, 16] state entering every tile (m1_bwd_tile() tokens) from the chunk's zero start
    float* wck;     // [batch, tiles, dim] sum of Delta from the chunk's start to the same tokens
    float* bcq;     // [batch, L, 32] fp32 records of B and C (the lane-per-channel summary pass)
    int lane_sum;   // the summary pass runs one channel per lane (rows 16-byte aligned)
    int chunk_img;  // the chunk pass reads 32-token row images (lane_sum, bf16 inputs, L and chunk multiples of 32)
    int64_t batch, dim, L;
    int64_t chunk;  // tokens per chunk: a multiple of m1_bwd_tile(), at most m1_bwd_max_chunk()
    int64_t G;      // chunks
    int N;
    int softplus;
};
int m1_bwd_tile();
int m1_bwd_max_chunk();
int m1_bwd_channels_per_block();
size_t m1_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t L, int64_t G);
void m1_bwd_carve(BwdArgs& a, void* ws);
hipError_t launch_m1_bwd(const BwdArgs& a, int in_bf16, int out_bf16, hipStream_t stream);

// Mamba-2.
struct M2Args {
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* dt_bias;
    void* y;
    float* last;
    const float* h0;  // [batch, H, P, N] initial state, or NULL for zero
    float* ws_bc;     // [batch, L, G, 2, N] fp32 copy of B and C (interleaved per token)
    float* ws_state;  // [batch, H, P, chunks, N] chunk end states, then carries-in
    float* ws_w;      // [batch, H, chunks] chunk sums of Delta / ln2
    int64_t batch, L, H, P, G, N;
    int64_t chunk;
    int chunks;
    int softplus;
    int xcd_units;    // chunked matrix form: place the units of one batch on one XCD
};

int m2_waves_per_block(int64_t N);

// Mamba-2 gradients (recurrent form, headdim 64).  Tensors as in selscan.h;
// ck, pB, pC, pA, pD, pbias point into the workspace (m2_bwd_carve).
struct M2BwdArgs {
    const void* x;
    const void* dt;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* dt_bias;
    const float* h0;
    const void* dout;
    float *dx, *ddt, *dA, *dB, *dC, *dD, *dz, *ddt_bias, *dh0;
    float* ck;        // [batch*H, tiles, N/16, 4, 64, 4] states entering each 8-token tile
                      // (the chunked form: each 32-token chunk, as
                      // [batch*H, chunks, N/16, 4, 4, 16, 4]: n block, p block,
                      // p quad, n in block, 4 consecutive p)
    float* pB;        // [batch*H, L, N] per-head dB
    float* pC;        // [batch*H, L, N] per-head dC
    float *pA, *pD, *pbias;   // [batch*H] per-(batch, head) sums
    int64_t batch, L, H, G, N;
    int softplus;
    int in_bf16;
};
size_t m2_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t N);
void m2_bwd_carve(M2BwdArgs& a, void* ws);
// ssd: the chunked matrix form (bf16 inputs, N in {32, 64, 128}, 16-byte aligned
// x, z, dout, B, C); otherwise the recurrent form
hipError_t launch_m2_bwd(const M2BwdArgs& a, int in_bf16, int out_bf16, int ssd, hipStream_t stream);

// One-token state update (decoding), both variants.  Mamba-1: u, delta, z, y
// [batch, dim]; B, C [batch, N]; A [dim, N]; D, bias [dim]; state
// [batch, dim, N].  Mamba-2: u = x, z, y [batch, H, P]; delta = dt
// [batch, H]; B, C [batch, G, N]; A, D, bias [H]; state [batch, H, P, N].
struct StepArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* bias;
    void* y;
    float* state;
    int64_t batch, dim;       // Mamba-1
    int64_t H, P, G;          // Mamba-2
    int N;
    int softplus;
    int vec;                  // A (16 bytes), B and C (4 elements) aligned for vector loads
};
hipError_t launch_step(const StepArgs& a, int in_bf16, int out_bf16, int mamba2, hipStream_t stream);

// Causal depthwise convolution: x, out [batch, dim, L]; w [dim, K]; bias [dim].
struct ConvArgs {
    const void* x;
    const float* w;
    const float* bias;
    void* out;
    int64_t batch, dim, L;
    int K;
    int silu;
    int vec_ok;   // L % 8 == 0 and 16-byte aligned rows of x and out
};
hipError_t launch_conv1d(const ConvArgs& a, int in_bf16, int out_bf16, hipStream_t stream);
hipError_t launch_m2(const M2Args& a, int in_bf16, int out_bf16, hipStream_t stream);
// Chunked matrix (SSD) form on MFMA for bf16 inputs, P = 64, N in {64, 128}.
bool m2_ssd_supported(const M2Args& a, int in_bf16);
// ws: 1 = warp-specialised kernel (state waves and chunk waves), 0 = every wave in every phase
hipError_t launch_m2_ssd(const M2Args& a, int out_bf16, int ws, hipStream_t stream);

}  // namespace selscan
