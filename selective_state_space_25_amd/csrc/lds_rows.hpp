// lds_rows.hpp -- 32-token tiles of 64 rows copied straight into LDS, for
// kernels whose wave gives each lane one row (channel) of [rows][L] tensors.
//
// One global_load_lds_dwordx4 fills 1 KB of LDS with 16 rows x 64 bytes (four
// consecutive 16-byte pieces of each row), so a row's share of a tile leaves
// as one memory request.  Lane i of instruction (h, k) takes row 16k + i%16,
// piece 4h + i/16 (h > 0 only for 4-byte elements, whose rows hold 8 pieces
// per tile).  Per tensor the LDS image is [h][k][p4][r] in 16-byte slots, and
// lane l finds piece p of its own row at slot (p/4) 256 + (p%4) 16 +
// (l/16) 64 + l%16: 16 consecutive lanes read 256 contiguous bytes, free of
// bank conflicts.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace selscan {
namespace rows {

typedef __attribute__((address_space(3))) void* ldsptr;

// 16-byte pieces per row in a 32-token tile of element type T.
template <typename T> constexpr int kPieces = 2 * (int)sizeof(T);

// lgkmcnt(0), vmcnt and expcnt left at their maxima
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// vmcnt(0), the others left at their maxima
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
}

// A pointer whose value is the same in every lane, held in SGPRs.
template <typename T>
__device__ __forceinline__ const T* uniform(const T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// 16 bytes per lane from g + OFF into LDS at slot + 16 * lane.  The
// instruction's immediate offset moves both the global and the LDS address,
// so M0 is set OFF bytes short of the slot; the immediate is 13-bit signed
// and larger offsets would wrap silently, so it is kept below 4096.
template <int OFF>
__device__ __forceinline__ void dma_at(const void* g, uint32_t slot) {
    static_assert(OFF >= 0 && OFF < 4096, "immediate offset out of range");
    __builtin_amdgcn_global_load_lds(g, (ldsptr)(uintptr_t)(slot - OFF), 16, OFF, 0);
}

// Addresses of the row copies of up to three tensors of element type T with
// the same row length L.  Rows past the block's last real row read that row
// (their values are never stored).  Both offsets stay below 64 rows x L x 4
// bytes, under 2^32 for L < 2^24.
template <typename T>
struct RowDma {
    const char* base[3];   // per tensor: the block's first row (wave-uniform)
    uint32_t kb[4];        // per row group k: byte offset of its first row (clamped)
    uint32_t voff[4];      // per row group: this lane's row and piece, from kb[k]

    // p[t]: tensor t's first row of the block; last: index of the block's
    // last real row (0..63)
    __device__ void init(const T* p0, const T* p1, const T* p2, int64_t L, int last, int lane) {
        base[0] = reinterpret_cast<const char*>(uniform(p0));
        base[1] = reinterpret_cast<const char*>(uniform(p1));
        base[2] = reinterpret_cast<const char*>(uniform(p2));
        const uint32_t rb = (uint32_t)(L * (int64_t)sizeof(T));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int k0 = min(16 * k, last);
            kb[k] = (uint32_t)k0 * rb;
            voff[k] = (uint32_t)min(lane & 15, last - k0) * rb + 16u * (uint32_t)(lane >> 4);
        }
    }
};

// Tokens t0 .. t0 + 31 of tensors 0 .. NT-1; tensor t lands at
// lds_base + t * kPieces<T> KB.
template <typename T, int NT>
__device__ __forceinline__ void issue_rows(const RowDma<T>& R, int64_t t0, uint32_t lds_base) {
    constexpr int NP = kPieces<T>;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const char* bt = R.base[t] + t0 * (int64_t)sizeof(T);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const char* g = bt + R.kb[k] + R.voff[k];
            const uint32_t s0 = lds_base + (uint32_t)(t * NP + k) * 1024u;
            dma_at<0>(g, s0);
            if constexpr (NP == 8) dma_at<64>(g, s0 + 4 * 1024u);
        }
    }
}

// This lane's slot offset within a tensor's image.
__device__ __forceinline__ int lane_slot(int lane) { return (lane >> 4) * 64 + (lane & 15); }

// 16-byte slot of piece p of tensor t (images of kPieces<T> KB each) for the
// lane whose slot offset is ls.
template <typename T>
__device__ __forceinline__ int piece_slot(int t, int p, int ls) {
    return t * kPieces<T> * 64 + (p >> 2) * 256 + (p & 3) * 16 + ls;
}

}  // namespace rows
}  // namespace selscan
