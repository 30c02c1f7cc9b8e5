// selscan.cpp -- host side of libselscan: argument checks, launch plans,
// workspace and error reporting behind the C ABI declared in selscan.h.
#include "selscan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "kernels.hpp"

namespace {

thread_local std::string g_error;

selscan_status_t fail(selscan_status_t s, const std::string& msg) {
    g_error = msg;
    return s;
}

selscan_status_t ok() {
    g_error.clear();
    return SELSCAN_OK;
}

int64_t env_int(const char* name, int64_t dflt) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::strtoll(v, nullptr, 10);
}

bool log_plans() { return env_int("SELSCAN_LOG", 0) != 0; }

// Compute units of the current device (256 on MI355X); cached per device.
int device_cus() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(mu);
    if (!cache[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

// Overflow-checked product of non-negative sizes; -1 on overflow.
int64_t mul_checked(std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x < 0) return -1;
        if (x != 0 && r > INT64_MAX / x) return -1;
        r *= x;
    }
    return r;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The current device must be a gfx950.  The architecture check runs once per
// device (cached like device_cus()); later calls only read the current device.
selscan_status_t device_check() {
    static std::mutex mu;
    static signed char arch_state[64] = {0};   // 0 unknown, 1 gfx950, -1 other
    static std::string other[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(SELSCAN_ERR_NO_DEVICE, "no HIP device available");
    if (dev < 64) {
        std::lock_guard<std::mutex> lk(mu);
        if (arch_state[dev] == 1) return SELSCAN_OK;
        if (arch_state[dev] == -1)
            return fail(SELSCAN_ERR_NO_DEVICE, "libselscan is built for gfx950, device is " + other[dev]);
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(SELSCAN_ERR_NO_DEVICE, "cannot query the HIP device");
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) {
        std::lock_guard<std::mutex> lk(mu);
        arch_state[dev] = ok ? 1 : -1;
        if (!ok) other[dev] = prop.gcnArchName;
    }
    if (!ok)
        return fail(SELSCAN_ERR_NO_DEVICE, std::string("libselscan is built for gfx950, device is ") +
                                               prop.gcnArchName);
    return SELSCAN_OK;
}

// ----------------------------------------------------------------- Mamba-1
struct M1Plan {
    int G;
    int xcd;   // chunk g on XCD g % 8 (G a multiple of 8)
    int carry_scan;   // carries from the scan kernel rather than a fold per chunk
    int64_t chunk;
    int NS;
    size_t bc_bytes, state_bytes, w_bytes, ws_bytes;
};

selscan_status_t check_m1_shape(const selscan_shape_t* s) {
    if (!s) return fail(SELSCAN_ERR_INVALID_ARG, "shape is NULL");
    if (s->batch < 1 || s->dim < 1 || s->seqlen < 1 || s->dstate < 1)
        return fail(SELSCAN_ERR_INVALID_ARG, "batch, dim, dstate and seqlen must all be >= 1");
    if (s->dstate > 16) return fail(SELSCAN_ERR_UNSUPPORTED, "Mamba-1 scan supports dstate <= 16");
    if ((s->in_dtype != SELSCAN_F32 && s->in_dtype != SELSCAN_BF16) ||
        (s->out_dtype != SELSCAN_F32 && s->out_dtype != SELSCAN_BF16))
        return fail(SELSCAN_ERR_UNSUPPORTED, "dtypes must be SELSCAN_F32 or SELSCAN_BF16");
    if (mul_checked({s->batch, s->dim, s->seqlen, 4}) < 0 || mul_checked({s->batch, s->dstate, s->seqlen, 4}) < 0 ||
        mul_checked({s->batch, s->dim, 64, 4}) < 0)
        return fail(SELSCAN_ERR_INVALID_ARG, "tensor sizes overflow 64-bit byte counts");
    if (s->batch * ((s->dim + 63) / 64) > 0x7fffffff || s->batch * ((s->seqlen + 31) / 32) > 0x7fffffff)
        return fail(SELSCAN_ERR_UNSUPPORTED, "too many channel blocks or token tiles for one launch");
    // the scan addresses a block's 64 rows with 32-bit byte offsets, and the
    // buffer descriptor of its y stores spans 64 rows of fp32 y: 64 L 4 bytes
    // stay below 2^32 only for L < 2^24
    if (s->seqlen >= (int64_t(1) << 24)) return fail(SELSCAN_ERR_UNSUPPORTED, "Mamba-1 scan supports seqlen < 2^24");
    return SELSCAN_OK;
}

M1Plan plan_m1(const selscan_shape_t* s) {
    M1Plan p;
    p.NS = selscan::m1_padded_states((int)s->dstate);
    const int64_t rows_pb = selscan::m1_rows_per_block();
    const int64_t wgs = s->batch * ((s->dim + rows_pb - 1) / rows_pb);
    const int64_t waves_per_chunk = wgs * selscan::m1_waves_per_block();
    int64_t G = env_int("SELSCAN_M1_CHUNKS", 0);
    if (G <= 0) {
        // one round of resident output-pass waves; rounding down avoids a
        // ragged last round
        const int64_t target = env_int(
            "SELSCAN_M1_WAVES",
            (int64_t)device_cus() * selscan::m1_resident_waves_per_cu(s->in_dtype == SELSCAN_BF16));
        G = std::max<int64_t>(1, target / waves_per_chunk);
        G = std::min<int64_t>(G, std::max<int64_t>(1, s->seqlen / 128));
        // whole groups of 8 chunks let each XCD own the chunks it scans,
        // unless rounding down to them gives up more than a tenth of the waves
        if (G >= 8 && (G / 8 * 8) * 10 >= G * 9) G = G / 8 * 8;
    }
    const int64_t align = selscan::m1_chunk_align(s->in_dtype == SELSCAN_BF16);
    G = std::max<int64_t>(1, std::min<int64_t>(G, (s->seqlen + align - 1) / align));
    G = std::min<int64_t>(G, 65535);
    // the kernels split the row's tiles as evenly as they can: the first
    // (tiles mod G) chunks take one tile more; chunk is the longest
    const int64_t tiles = (s->seqlen + align - 1) / align;
    const int64_t chunk = (tiles + G - 1) / G * align;
    p.G = (int)G;
    p.chunk = chunk;
    p.xcd = G % 8 == 0 && wgs * G < (int64_t(1) << 24) && env_int("SELSCAN_M1_XCD", 1) != 0;
    // chunk g folds the g summaries before it at its start: hidden behind the
    // scan up to about 16 chunks (measured), beyond that the fold's latency
    // grows into the output pass and one scan over all summaries (a launch of
    // its own, 20-35 us on Mamba-130m/2.8b-sized layers) is cheaper
    p.carry_scan = G > 1 && env_int("SELSCAN_M1_CARRY_SCAN", G > 16 ? 1 : 0) != 0;
    const int64_t rows = s->batch * s->dim;
    p.bc_bytes = align256(selscan::m1_bc_bytes(s->batch, s->seqlen));
    p.state_bytes = G > 1 ? align256((size_t)rows * G * p.NS * 4) : 0;
    p.w_bytes = G > 1 ? align256((size_t)rows * G * 4) : 0;
    p.ws_bytes = p.bc_bytes + p.state_bytes + p.w_bytes;
    return p;
}

// ----------------------------------------------------------------- Mamba-2
struct M2Plan {
    int chunks;
    int64_t chunk;
    size_t bc_bytes, state_bytes, w_bytes, ws_bytes;
};

selscan_status_t check_m2_shape(const selscan_m2_shape_t* s) {
    if (!s) return fail(SELSCAN_ERR_INVALID_ARG, "shape is NULL");
    if (s->batch < 1 || s->seqlen < 1 || s->nheads < 1 || s->headdim < 1 || s->ngroups < 1 || s->dstate < 1)
        return fail(SELSCAN_ERR_INVALID_ARG, "batch, seqlen, nheads, headdim, ngroups, dstate must be >= 1");
    if (s->nheads % s->ngroups != 0) return fail(SELSCAN_ERR_INVALID_ARG, "nheads must be a multiple of ngroups");
    if (s->dstate != 16 && s->dstate != 32 && s->dstate != 64 && s->dstate != 128)
        return fail(SELSCAN_ERR_UNSUPPORTED, "Mamba-2 scan supports dstate 16, 32, 64, 128");
    if ((s->in_dtype != SELSCAN_F32 && s->in_dtype != SELSCAN_BF16) ||
        (s->out_dtype != SELSCAN_F32 && s->out_dtype != SELSCAN_BF16))
        return fail(SELSCAN_ERR_UNSUPPORTED, "dtypes must be SELSCAN_F32 or SELSCAN_BF16");
    if (mul_checked({s->batch, s->seqlen, s->nheads, s->headdim, 4}) < 0 ||
        mul_checked({s->batch, s->seqlen, s->ngroups, s->dstate, 8}) < 0 ||
        mul_checked({s->batch, s->nheads, s->headdim, s->dstate, 4, 1024}) < 0)
        return fail(SELSCAN_ERR_INVALID_ARG, "tensor sizes overflow 64-bit byte counts");
    if (s->batch * s->nheads * ((s->headdim + 63) / 64) > 0x7fffffff)
        return fail(SELSCAN_ERR_UNSUPPORTED, "too many (batch, head) units for one launch");
    return SELSCAN_OK;
}

M2Plan plan_m2(const selscan_m2_shape_t* s) {
    M2Plan p;
    const int64_t waves = s->batch * s->nheads * ((s->headdim + 63) / 64) * selscan::m2_waves_per_block(s->dstate);
    int64_t G = env_int("SELSCAN_M2_CHUNKS", 0);
    if (G <= 0) {
        const int64_t target = env_int("SELSCAN_M2_WAVES", (int64_t)device_cus() * 8);
        G = (target + waves - 1) / waves;
        G = std::min<int64_t>(G, std::max<int64_t>(1, s->seqlen / 64));
    }
    G = std::max<int64_t>(1, std::min<int64_t>(G, s->seqlen));
    G = std::min<int64_t>(G, 65535);
    int64_t chunk = (s->seqlen + G - 1) / G;
    G = (s->seqlen + chunk - 1) / chunk;
    p.chunks = (int)G;
    p.chunk = chunk;
    p.bc_bytes = align256((size_t)s->batch * s->seqlen * s->ngroups * 2 * s->dstate * 4);
    if (G > 1) {
        p.state_bytes = align256((size_t)s->batch * s->nheads * s->headdim * G * s->dstate * 4);
        p.w_bytes = align256((size_t)s->batch * s->nheads * G * 4);
    } else {
        p.state_bytes = p.w_bytes = 0;
    }
    p.ws_bytes = p.bc_bytes + p.state_bytes + p.w_bytes;
    return p;
}

// Stream-ordered scratch: the caller's workspace when given, else an
// allocation freed on the same stream after the launches.
struct Scratch {
    void* ptr = nullptr;
    bool owned = false;
    hipStream_t stream = nullptr;
    selscan_status_t get(void* user, size_t user_bytes, size_t need, hipStream_t st) {
        stream = st;
        if (need == 0) return SELSCAN_OK;
        if (user) {
            if (user_bytes < need)
                return fail(SELSCAN_ERR_WORKSPACE, "workspace is smaller than the required " + std::to_string(need) +
                                                       " bytes");
            if ((reinterpret_cast<uintptr_t>(user) & 255) != 0)
                return fail(SELSCAN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
            ptr = user;
            return SELSCAN_OK;
        }
        if (hipMallocAsync(&ptr, need, st) != hipSuccess) {
            (void)hipGetLastError();
            return fail(SELSCAN_ERR_LAUNCH, "hipMallocAsync of " + std::to_string(need) + " workspace bytes failed");
        }
        owned = true;
        return SELSCAN_OK;
    }
    void release() {
        if (owned && ptr) (void)hipFreeAsync(ptr, stream);
        ptr = nullptr;
        owned = false;
    }
};

// ------------------------------------------------------- Mamba-1 backward
struct BwdPlan {
    int64_t chunk, G;
    size_t ws_bytes;
};

BwdPlan plan_m1_bwd(const selscan_shape_t* s) {
    BwdPlan p;
    const int64_t tile = selscan::m1_bwd_tile();
    const int64_t nbc = (s->dim + selscan::m1_bwd_channels_per_block() - 1) / selscan::m1_bwd_channels_per_block();
    int64_t chunk = env_int("SELSCAN_BWD_CHUNK", 0);
    if (chunk <= 0) {
        // the longest chunk that still gives every compute unit eight
        // workgroups of 64 channels (two to eight are resident per unit,
        // depending on the pass)
        chunk = selscan::m1_bwd_max_chunk();
        const int64_t want = 8 * (int64_t)device_cus();
        while (chunk > 2 * tile && s->batch * nbc * ((s->seqlen + chunk - 1) / chunk) < want) chunk /= 2;
    }
    chunk = std::min<int64_t>(std::max<int64_t>(tile, (chunk + tile - 1) / tile * tile), selscan::m1_bwd_max_chunk());
    p.chunk = chunk;
    p.G = (s->seqlen + chunk - 1) / chunk;
    p.ws_bytes = selscan::m1_bwd_workspace_bytes(s->batch, s->dim, s->seqlen, p.G);
    return p;
}

selscan_status_t check_m1_bwd_shape(const selscan_shape_t* s) {
    selscan_status_t st = check_m1_shape(s);
    if (st != SELSCAN_OK) return st;
    // per-thread byte offsets within a workgroup's rows are 32-bit
    if (s->seqlen > (int64_t(1) << 22)) return fail(SELSCAN_ERR_UNSUPPORTED, "Mamba-1 backward supports seqlen <= 2^22");
    const int64_t nbc = (s->dim + selscan::m1_bwd_channels_per_block() - 1) / selscan::m1_bwd_channels_per_block();
    const int64_t tiles = (s->seqlen + selscan::m1_bwd_tile() - 1) / selscan::m1_bwd_tile();
    if (mul_checked({nbc, s->batch, 32, s->seqlen, 4}) < 0 || mul_checked({s->batch, s->dim, tiles, 17, 4}) < 0)
        return fail(SELSCAN_ERR_INVALID_ARG, "workspace size overflows 64-bit byte counts");
    if (s->batch * nbc * tiles > 0x7fffffff)
        return fail(SELSCAN_ERR_UNSUPPORTED, "too many workgroups for one launch");
    return SELSCAN_OK;
}

}  // namespace

selscan_status_t selscan::set_error(selscan_status_t s, const std::string& msg) { return fail(s, msg); }

extern "C" {

const char* selscan_last_error(void) { return g_error.c_str(); }

const char* selscan_version(void) { return "libselscan 0.1 gfx950"; }

size_t selscan_workspace_bytes(const selscan_shape_t* shape) {
    if (check_m1_shape(shape) != SELSCAN_OK) return 0;
    return plan_m1(shape).ws_bytes;
}

size_t selscan_bwd_workspace_bytes(const selscan_shape_t* shape) {
    if (check_m1_bwd_shape(shape) != SELSCAN_OK) return 0;
    return plan_m1_bwd(shape).ws_bytes;
}

size_t selscan_mamba2_workspace_bytes(const selscan_m2_shape_t* shape) {
    if (check_m2_shape(shape) != SELSCAN_OK) return 0;
    return plan_m2(shape).ws_bytes;
}

selscan_status_t selscan_fwd(const selscan_shape_t* s, const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z,
                             const float* delta_bias, int softplus, void* y, float* last_state, void* stream) {
    return selscan_fwd_h0(s, u, delta, A, B, C, D, z, delta_bias, softplus, nullptr, y, last_state, stream);
}

selscan_status_t selscan_fwd_h0(const selscan_shape_t* s, const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, int softplus, const float* h0, void* y, float* last_state,
                                void* stream) {
    try {
        selscan_status_t st = check_m1_shape(s);
        if (st != SELSCAN_OK) return st;
        if (!u || !delta || !A || !B || !C || !y)
            return fail(SELSCAN_ERR_INVALID_ARG, "u, delta, A, B, C and y must be non-NULL");
        if (softplus != 0 && softplus != 1) return fail(SELSCAN_ERR_INVALID_ARG, "softplus must be 0 or 1");
        if (h0 && last_state && static_cast<const void*>(h0) == static_cast<const void*>(last_state))
            return fail(SELSCAN_ERR_INVALID_ARG, "h0 and last_state must not alias");
        st = device_check();
        if (st != SELSCAN_OK) return st;
        const M1Plan plan = plan_m1(s);
        hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
        Scratch ws;
        st = ws.get(s->workspace, s->workspace_bytes, plan.ws_bytes, hs);
        if (st != SELSCAN_OK) return st;

        const int in_bf16 = s->in_dtype == SELSCAN_BF16;
        const int out_bf16 = s->out_dtype == SELSCAN_BF16;
        const int64_t in_es = in_bf16 ? 2 : 4, out_es = out_bf16 ? 2 : 4;
        selscan::M1Args a{};
        a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
        a.y = y; a.last = last_state; a.h0 = h0;
        a.batch = s->batch; a.dim = s->dim; a.L = s->seqlen; a.N = (int)s->dstate;
        a.G = plan.G; a.chunk = plan.chunk; a.softplus = softplus;
        a.force_general = env_int("SELSCAN_FORCE_GENERAL", 0) != 0;
        a.xcd_chunks = plan.xcd;
        a.carry_scan = plan.carry_scan;
        // 32-token runs of every row start on 16-byte boundaries
        a.vec_ok = (s->seqlen * in_es) % 16 == 0 && (s->seqlen * out_es) % 16 == 0 && aligned16(u) &&
                   aligned16(delta) && aligned16(y) && (!z || aligned16(z));
        char* base = static_cast<char*>(ws.ptr);
        a.bcq = reinterpret_cast<float*>(base);
        if (plan.G > 1) {
            a.ws_state = reinterpret_cast<float*>(base + plan.bc_bytes);
            a.ws_w = reinterpret_cast<float*>(base + plan.bc_bytes + plan.state_bytes);
        }
        if (log_plans())
            std::fprintf(stderr, "[selscan] m1 B=%lld D=%lld N=%lld L=%lld chunks=%d chunk=%lld ws=%zu vec=%d xcd=%d scan=%d\n",
                         (long long)s->batch, (long long)s->dim, (long long)s->dstate, (long long)s->seqlen, plan.G,
                         (long long)plan.chunk, plan.ws_bytes, a.vec_ok, a.xcd_chunks, a.carry_scan);
        hipError_t e = selscan::launch_m1(a, in_bf16, out_bf16, hs);
        ws.release();
        if (e != hipSuccess) return fail(SELSCAN_ERR_LAUNCH, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(SELSCAN_ERR_LAUNCH, "unexpected host exception");
    }
}

selscan_status_t selscan_mamba2_fwd(const selscan_m2_shape_t* s, const void* x, const void* dt, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    const float* dt_bias, int softplus, void* y, float* last_state, void* stream) {
    return selscan_mamba2_fwd_h0(s, x, dt, A, B, C, D, z, dt_bias, softplus, nullptr, y, last_state, stream);
}

selscan_status_t selscan_mamba2_fwd_h0(const selscan_m2_shape_t* s, const void* x, const void* dt, const float* A,
                                       const void* B, const void* C, const float* D, const void* z,
                                       const float* dt_bias, int softplus, const float* h0, void* y,
                                       float* last_state, void* stream) {
    try {
        selscan_status_t st = check_m2_shape(s);
        if (st != SELSCAN_OK) return st;
        if (!x || !dt || !A || !B || !C || !y)
            return fail(SELSCAN_ERR_INVALID_ARG, "x, dt, A, B, C and y must be non-NULL");
        if (softplus != 0 && softplus != 1) return fail(SELSCAN_ERR_INVALID_ARG, "softplus must be 0 or 1");
        if (h0 && last_state && static_cast<const void*>(h0) == static_cast<const void*>(last_state))
            return fail(SELSCAN_ERR_INVALID_ARG, "h0 and last_state must not alias");
        st = device_check();
        if (st != SELSCAN_OK) return st;
        const M2Plan plan = plan_m2(s);
        hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
        selscan::M2Args a{};
        a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.dt_bias = dt_bias;
        a.y = y; a.last = last_state; a.h0 = h0;
        a.batch = s->batch; a.L = s->seqlen; a.H = s->nheads; a.P = s->headdim; a.G = s->ngroups; a.N = s->dstate;
        a.chunks = plan.chunks; a.chunk = plan.chunk; a.softplus = softplus;
        const int in_bf16 = s->in_dtype == SELSCAN_BF16, out_bf16 = s->out_dtype == SELSCAN_BF16;
        if (env_int("SELSCAN_M2_SSD", 1) != 0 && selscan::m2_ssd_supported(a, in_bf16) && aligned16(x) &&
            aligned16(B) && aligned16(C)) {
            // chunked matrix form on MFMA; needs no workspace
            const int ws_form = env_int("SELSCAN_M2_SSD_WS", 1) != 0;
            a.xcd_units = env_int("SELSCAN_M2_XCD_UNITS", 1) != 0;
            if (log_plans())
                std::fprintf(stderr, "[selscan] m2 ssd B=%lld L=%lld H=%lld P=%lld G=%lld N=%lld ws=%d\n",
                             (long long)s->batch, (long long)s->seqlen, (long long)s->nheads, (long long)s->headdim,
                             (long long)s->ngroups, (long long)s->dstate, ws_form);
            hipError_t e = selscan::launch_m2_ssd(a, out_bf16, ws_form, hs);
            if (e != hipSuccess)
                return fail(SELSCAN_ERR_LAUNCH, std::string("kernel launch failed: ") + hipGetErrorString(e));
            return ok();
        }
        Scratch ws;
        st = ws.get(s->workspace, s->workspace_bytes, plan.ws_bytes, hs);
        if (st != SELSCAN_OK) return st;
        char* base = static_cast<char*>(ws.ptr);
        a.ws_bc = reinterpret_cast<float*>(base);
        if (plan.chunks > 1) {
            a.ws_state = reinterpret_cast<float*>(base + plan.bc_bytes);
            a.ws_w = reinterpret_cast<float*>(base + plan.bc_bytes + plan.state_bytes);
        }
        if (log_plans())
            std::fprintf(stderr, "[selscan] m2 B=%lld L=%lld H=%lld P=%lld G=%lld N=%lld chunks=%d chunk=%lld ws=%zu\n",
                         (long long)s->batch, (long long)s->seqlen, (long long)s->nheads, (long long)s->headdim,
                         (long long)s->ngroups, (long long)s->dstate, plan.chunks, (long long)plan.chunk,
                         plan.ws_bytes);
        hipError_t e = selscan::launch_m2(a, in_bf16, out_bf16, hs);
        ws.release();
        if (e != hipSuccess) return fail(SELSCAN_ERR_LAUNCH, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(SELSCAN_ERR_LAUNCH, "unexpected host exception");
    }
}

selscan_status_t selscan_step(const selscan_shape_t* s, float* state, const void* u, const void* delta,
                              const float* A, const void* B, const void* C, const float* D, const void* z,
                              const float* delta_bias, int softplus, void* y, void* stream) {
    try {
        if (!s) return fail(SELSCAN_ERR_INVALID_ARG, "shape is NULL");
        if (s->batch < 1 || s->dim < 1 || s->dstate < 1)
            return fail(SELSCAN_ERR_INVALID_ARG, "batch, dim and dstate must all be >= 1");
        if (s->dstate > 16) return fail(SELSCAN_ERR_UNSUPPORTED, "Mamba-1 step supports dstate <= 16");
        if ((s->in_dtype != SELSCAN_F32 && s->in_dtype != SELSCAN_BF16) ||
            (s->out_dtype != SELSCAN_F32 && s->out_dtype != SELSCAN_BF16))
            return fail(SELSCAN_ERR_UNSUPPORTED, "dtypes must be SELSCAN_F32 or SELSCAN_BF16");
        if (mul_checked({s->batch, s->dim, s->dstate, 4}) < 0)
            return fail(SELSCAN_ERR_INVALID_ARG, "tensor sizes overflow 64-bit byte counts");
        if (!state || !u || !delta || !A || !B || !C || !y)
            return fail(SELSCAN_ERR_INVALID_ARG, "state, u, delta, A, B, C and y must be non-NULL");
        if (s->dstate % 4 == 0 && !aligned16(state))
            return fail(SELSCAN_ERR_INVALID_ARG, "state must be 16-byte aligned");
        if (softplus != 0 && softplus != 1) return fail(SELSCAN_ERR_INVALID_ARG, "softplus must be 0 or 1");
        selscan_status_t st = device_check();
        if (st != SELSCAN_OK) return st;
        selscan::StepArgs a{};
        a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
        a.y = y; a.state = state;
        a.batch = s->batch; a.dim = s->dim; a.N = (int)s->dstate; a.softplus = softplus;
        const uintptr_t v4 = s->in_dtype == SELSCAN_BF16 ? 8 : 16;   // bytes of 4 input elements
        a.vec = aligned16(A) && (reinterpret_cast<uintptr_t>(B) % v4) == 0 && (reinterpret_cast<uintptr_t>(C) % v4) == 0;
        hipError_t e = selscan::launch_step(a, s->in_dtype == SELSCAN_BF16, s->out_dtype == SELSCAN_BF16, 0,
                                            reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(SELSCAN_ERR_LAUNCH, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(SELSCAN_ERR_LAUNCH, "unexpected host exception");
    }
}

selscan_status_t selscan_bwd(const selscan_shape_t* s, const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z, const float* delta_bias,
                             int softplus, const float* h0, const void* dout, float* du, float* ddelta, float* dA,
                             float* dB, float* dC, float* dD, float* dz, float* ddelta_bias, float* dh0,
                             void* stream) {
    try {
        selscan_status_t st = check_m1_bwd_shape(s);
        if (st != SELSCAN_OK) return st;
        if (!u || !delta || !A || !B || !C || !dout)
            return fail(SELSCAN_ERR_INVALID_ARG, "u, delta, A, B, C and dout must be non-NULL");
        if (!du || !ddelta || !dA || !dB || !dC)
            return fail(SELSCAN_ERR_INVALID_ARG, "du, ddelta, dA, dB and dC must be non-NULL");
        if (z && !dz) return fail(SELSCAN_ERR_INVALID_ARG, "dz must be non-NULL when z is given");
        if (softplus != 0 && softplus != 1) return fail(SELSCAN_ERR_INVALID_ARG, "softplus must be 0 or 1");
        st = device_check();
        if (st != SELSCAN_OK) return st;
        const BwdPlan plan = plan_m1_bwd(s);
        hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
        Scratch ws;
        st = ws.get(s->workspace, s->workspace_bytes, plan.ws_bytes, hs);
        if (st != SELSCAN_OK) return st;
        selscan::BwdArgs a{};
        a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias; a.h0 = h0;
        a.dout = dout;
        a.du = du; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.dz = dz;
        a.dbias = ddelta_bias; a.dh0 = dh0;
        a.batch = s->batch; a.dim = s->dim; a.L = s->seqlen; a.N = (int)s->dstate; a.softplus = softplus;
        a.chunk = plan.chunk; a.G = plan.G;
        {   // rows on 16-byte boundaries: the summary pass runs one channel per lane
            const int64_t si = s->in_dtype == SELSCAN_BF16 ? 2 : 4, so = s->out_dtype == SELSCAN_BF16 ? 2 : 4;
            a.lane_sum = aligned16(u) && aligned16(delta) && (!z || aligned16(z)) && aligned16(dout) &&
                         (s->seqlen * si) % 16 == 0 && (s->seqlen * so) % 16 == 0 &&
                         env_int("SELSCAN_BWD_LANE_SUMMARY", 1) != 0;
            // (the row-image chunk pass also stores 16 bytes per row at a time)
            a.chunk_img = a.lane_sum && s->in_dtype == SELSCAN_BF16 && s->seqlen % 32 == 0 && plan.chunk % 32 == 0 &&
                          aligned16(du) && aligned16(ddelta) && (!dz || aligned16(dz)) &&
                          env_int("SELSCAN_BWD_CHUNK_IMAGES", 1) != 0;
        }
        selscan::m1_bwd_carve(a, ws.ptr);
        if (log_plans())
            std::fprintf(stderr, "[selscan] m1 bwd B=%lld D=%lld N=%lld L=%lld chunks=%lld chunk=%lld ws=%zu lane_sum=%d\n",
                         (long long)s->batch, (long long)s->dim, (long long)s->dstate, (long long)s->seqlen,
                         (long long)plan.G, (long long)plan.chunk, plan.ws_bytes, a.lane_sum);
        hipError_t e = selscan::launch_m1_bwd(a, s->in_dtype == SELSCAN_BF16, s->out_dtype == SELSCAN_BF16, hs);
        ws.release();
        if (e != hipSuccess) return fail(SELSCAN_ERR_LAUNCH, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(SELSCAN_ERR_LAUNCH, "unexpected host exception");
    }
}

// Mamba-2 gradients: the recurrent form with lane = channel needs headdim 64.
selscan_status_t check_m2_bwd_shape(const selscan_m2_shape_t* s) {
    selscan_status_t st = check_m2_shape(s);
    if (st != SELSCAN_OK) return st;
    if (s->headdim != 64) return fail(SELSCAN_ERR_UNSUPPORTED, "Mamba-2 gradients support headdim 64");
    if (s->batch * s->nheads > 0x7fffffff) return fail(SELSCAN_ERR_UNSUPPORTED, "too many (batch, head) units");
    if (s->batch * s->seqlen * s->ngroups * s->dstate > (int64_t)0xffffffff * 256)
        return fail(SELSCAN_ERR_UNSUPPORTED, "too many dB/dC elements for one launch");
    return SELSCAN_OK;
}

size_t selscan_mamba2_bwd_workspace_bytes(const selscan_m2_shape_t* s) {
    if (check_m2_bwd_shape(s) != SELSCAN_OK) return 0;
    return selscan::m2_bwd_workspace_bytes(s->batch, s->seqlen, s->nheads, s->dstate);
}

selscan_status_t selscan_mamba2_bwd(const selscan_m2_shape_t* s, const void* x, const void* dt, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    const float* dt_bias, int softplus, const float* h0, const void* dout,
                                    float* dx, float* ddt, float* dA, float* dB, float* dC, float* dD, float* dz,
                                    float* ddt_bias, float* dh0, void* stream) {
    try {
        selscan_status_t st = check_m2_bwd_shape(s);
        if (st != SELSCAN_OK) return st;
        if (!x || !dt || !A || !B || !C || !dout)
            return fail(SELSCAN_ERR_INVALID_ARG, "x, dt, A, B, C and dout must be non-NULL");
        if (!dx || !ddt || !dA || !dB || !dC)
            return fail(SELSCAN_ERR_INVALID_ARG, "dx, ddt, dA, dB and dC must be non-NULL");
        if (z && !dz) return fail(SELSCAN_ERR_INVALID_ARG, "dz must be non-NULL when z is given");
        if (softplus != 0 && softplus != 1) return fail(SELSCAN_ERR_INVALID_ARG, "softplus must be 0 or 1");
        st = device_check();
        if (st != SELSCAN_OK) return st;
        hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
        Scratch ws;
        st = ws.get(s->workspace, s->workspace_bytes,
                    selscan::m2_bwd_workspace_bytes(s->batch, s->seqlen, s->nheads, s->dstate), hs);
        if (st != SELSCAN_OK) return st;
        selscan::M2BwdArgs a{};
        a.x = x; a.dt = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.dt_bias = dt_bias; a.h0 = h0;
        a.dout = dout;
        a.dx = dx; a.ddt = ddt; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.dz = dz; a.ddt_bias = ddt_bias;
        a.dh0 = dh0;
        a.batch = s->batch; a.L = s->seqlen; a.H = s->nheads; a.G = s->ngroups; a.N = s->dstate;
        a.softplus = softplus;
        a.in_bf16 = s->in_dtype == SELSCAN_BF16;
        selscan::m2_bwd_carve(a, ws.ptr);
        if (log_plans())
            std::fprintf(stderr, "[selscan] m2 bwd B=%lld L=%lld H=%lld G=%lld N=%lld ws=%zu\n", (long long)s->batch,
                         (long long)s->seqlen, (long long)s->nheads, (long long)s->ngroups, (long long)s->dstate,
                         selscan::m2_bwd_workspace_bytes(s->batch, s->seqlen, s->nheads, s->dstate));
        hipError_t e = selscan::launch_m2_bwd(a, a.in_bf16, s->out_dtype == SELSCAN_BF16,
                                              env_int("SELSCAN_M2_BWD_SSD", 1) != 0, hs);
        ws.release();
        if (e != hipSuccess) return fail(SELSCAN_ERR_LAUNCH, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(SELSCAN_ERR_LAUNCH, "unexpected host exception");
    }
}

selscan_status_t selscan_mamba2_step(const selscan_m2_shape_t* s, float* state, const void* x, const void* dt,
                                     const float* A, const void* B, const void* C, const float* D, const void* z,
                                     const float* dt_bias, int softplus, void* y, void* stream) {
    try {
        if (!s) return fail(SELSCAN_ERR_INVALID_ARG, "shape is NULL");
        if (s->batch < 1 || s->nheads < 1 || s->headdim < 1 || s->ngroups < 1 || s->dstate < 1)
            return fail(SELSCAN_ERR_INVALID_ARG, "batch, nheads, headdim, ngroups, dstate must be >= 1");
        if (s->nheads % s->ngroups != 0) return fail(SELSCAN_ERR_INVALID_ARG, "nheads must be a multiple of ngroups");
        if (s->dstate != 16 && s->dstate != 32 && s->dstate != 64 && s->dstate != 128)
            return fail(SELSCAN_ERR_UNSUPPORTED, "Mamba-2 step supports dstate 16, 32, 64, 128");
        if ((s->in_dtype != SELSCAN_F32 && s->in_dtype != SELSCAN_BF16) ||
            (s->out_dtype != SELSCAN_F32 && s->out_dtype != SELSCAN_BF16))
            return fail(SELSCAN_ERR_UNSUPPORTED, "dtypes must be SELSCAN_F32 or SELSCAN_BF16");
        if (mul_checked({s->batch, s->nheads, s->headdim, s->dstate, 4}) < 0)
            return fail(SELSCAN_ERR_INVALID_ARG, "tensor sizes overflow 64-bit byte counts");
        if (!state || !x || !dt || !A || !B || !C || !y)
            return fail(SELSCAN_ERR_INVALID_ARG, "state, x, dt, A, B, C and y must be non-NULL");
        if (!aligned16(state)) return fail(SELSCAN_ERR_INVALID_ARG, "state must be 16-byte aligned");
        if (softplus != 0 && softplus != 1) return fail(SELSCAN_ERR_INVALID_ARG, "softplus must be 0 or 1");
        selscan_status_t st = device_check();
        if (st != SELSCAN_OK) return st;
        selscan::StepArgs a{};
        a.u = x; a.delta = dt; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = dt_bias;
        a.y = y; a.state = state;
        a.batch = s->batch; a.H = s->nheads; a.P = s->headdim; a.G = s->ngroups; a.N = (int)s->dstate;
        a.softplus = softplus;
        const uintptr_t v4 = s->in_dtype == SELSCAN_BF16 ? 8 : 16;   // bytes of 4 input elements
        a.vec = (reinterpret_cast<uintptr_t>(B) % v4) == 0 && (reinterpret_cast<uintptr_t>(C) % v4) == 0;
        hipError_t e = selscan::launch_step(a, s->in_dtype == SELSCAN_BF16, s->out_dtype == SELSCAN_BF16, 1,
                                            reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(SELSCAN_ERR_LAUNCH, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(SELSCAN_ERR_LAUNCH, "unexpected host exception");
    }
}

selscan_status_t selscan_conv1d(const selscan_conv_shape_t* s, const void* x, const float* weight,
                                const float* bias, int silu, void* out, void* stream) {
    try {
        if (!s) return fail(SELSCAN_ERR_INVALID_ARG, "shape is NULL");
        if (s->batch < 1 || s->dim < 1 || s->seqlen < 1 || s->width < 1)
            return fail(SELSCAN_ERR_INVALID_ARG, "batch, dim, seqlen and width must all be >= 1");
        if (s->width > 64) return fail(SELSCAN_ERR_UNSUPPORTED, "conv1d supports width <= 64");
        if ((s->in_dtype != SELSCAN_F32 && s->in_dtype != SELSCAN_BF16) ||
            (s->out_dtype != SELSCAN_F32 && s->out_dtype != SELSCAN_BF16))
            return fail(SELSCAN_ERR_UNSUPPORTED, "dtypes must be SELSCAN_F32 or SELSCAN_BF16");
        if (mul_checked({s->batch, s->dim, s->seqlen, 4}) < 0 || mul_checked({s->dim, s->width, 4}) < 0)
            return fail(SELSCAN_ERR_INVALID_ARG, "tensor sizes overflow 64-bit byte counts");
        if (!x || !weight || !out) return fail(SELSCAN_ERR_INVALID_ARG, "x, weight and out must be non-NULL");
        if (silu != 0 && silu != 1) return fail(SELSCAN_ERR_INVALID_ARG, "silu must be 0 or 1");
        if (x == out) return fail(SELSCAN_ERR_INVALID_ARG, "out must not alias x");
        selscan_status_t st = device_check();
        if (st != SELSCAN_OK) return st;
        const int in_bf16 = s->in_dtype == SELSCAN_BF16, out_bf16 = s->out_dtype == SELSCAN_BF16;
        selscan::ConvArgs a{};
        a.x = x; a.w = weight; a.bias = bias; a.out = out;
        a.batch = s->batch; a.dim = s->dim; a.L = s->seqlen; a.K = (int)s->width; a.silu = silu;
        a.vec_ok = s->seqlen % 8 == 0 && aligned16(x) && aligned16(out);
        hipError_t e = selscan::launch_conv1d(a, in_bf16, out_bf16, reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(SELSCAN_ERR_LAUNCH, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return ok();
    } catch (...) {
        return fail(SELSCAN_ERR_LAUNCH, "unexpected host exception");
    }
}

}  // extern "C"
