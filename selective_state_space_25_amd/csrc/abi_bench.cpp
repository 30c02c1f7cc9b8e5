// abi_bench -- host cost of the decode entry points, timed from C++.
//
// The one-token update is short enough (a few microseconds of GPU time)
// that the host's cost per call matters.  This program calls selscan_step
// and selscan_mamba2_step back to back on zero-filled device buffers at
// the decode shapes the benchmark uses (Mamba-1: batch 4, 5120 channels,
// 16 states; Mamba-2: batch 8, 32 heads of 64 channels, one group, 128
// states; bf16 inputs, fp32 state and y) and reports the host time per
// call: the C-ABI entry's checks plus the kernel launch, with no Python in
// the way.  Usage: abi_bench [calls]; prints one JSON line.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>

#include "selscan.h"

namespace {

void* dev_zeros(size_t bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess || hipMemset(p, 0, bytes) != hipSuccess) {
        std::fprintf(stderr, "abi_bench: device allocation of %zu bytes failed\n", bytes);
        std::exit(1);
    }
    return p;
}

void check(selscan_status_t s) {
    if (s != SELSCAN_OK) {
        std::fprintf(stderr, "abi_bench: call failed: %s\n", selscan_last_error());
        std::exit(1);
    }
}

template <typename F>
double host_us_per_call(F call, int calls) {
    for (int i = 0; i < 50; ++i) call();
    if (hipDeviceSynchronize() != hipSuccess) std::exit(1);
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < calls; ++i) call();
    const auto t1 = std::chrono::steady_clock::now();
    if (hipDeviceSynchronize() != hipSuccess) std::exit(1);
    return std::chrono::duration<double, std::micro>(t1 - t0).count() / calls;
}

}  // namespace

int main(int argc, char** argv) {
    const int calls = argc > 1 ? std::atoi(argv[1]) : 200;
    if (calls < 1) return 2;

    const int64_t b1 = 4, d1 = 5120, n1 = 16;
    selscan_shape_t s1{b1, d1, n1, 1, SELSCAN_BF16, SELSCAN_F32, nullptr, 0};
    float* state1 = static_cast<float*>(dev_zeros(b1 * d1 * n1 * 4));
    void* u = dev_zeros(b1 * d1 * 2);
    void* dl = dev_zeros(b1 * d1 * 2);
    void* z1 = dev_zeros(b1 * d1 * 2);
    float* A1 = static_cast<float*>(dev_zeros(d1 * n1 * 4));
    void* B1 = dev_zeros(b1 * n1 * 2);
    void* C1 = dev_zeros(b1 * n1 * 2);
    float* D1 = static_cast<float*>(dev_zeros(d1 * 4));
    float* bias1 = static_cast<float*>(dev_zeros(d1 * 4));
    void* y1 = dev_zeros(b1 * d1 * 4);
    const double m1 = host_us_per_call(
        [&] { check(selscan_step(&s1, state1, u, dl, A1, B1, C1, D1, z1, bias1, 1, y1, nullptr)); }, calls);

    const int64_t b2 = 8, h2 = 32, p2 = 64, g2 = 1, n2 = 128;
    selscan_m2_shape_t s2{b2, 1, h2, p2, g2, n2, SELSCAN_BF16, SELSCAN_F32, nullptr, 0};
    float* state2 = static_cast<float*>(dev_zeros(b2 * h2 * p2 * n2 * 4));
    void* x = dev_zeros(b2 * h2 * p2 * 2);
    void* z2 = dev_zeros(b2 * h2 * p2 * 2);
    void* dt = dev_zeros(b2 * h2 * 2);
    float* A2 = static_cast<float*>(dev_zeros(h2 * 4));
    void* B2 = dev_zeros(b2 * g2 * n2 * 2);
    void* C2 = dev_zeros(b2 * g2 * n2 * 2);
    float* D2 = static_cast<float*>(dev_zeros(h2 * 4));
    float* bias2 = static_cast<float*>(dev_zeros(h2 * 4));
    void* y2 = dev_zeros(b2 * h2 * p2 * 4);
    const double m2 = host_us_per_call(
        [&] { check(selscan_mamba2_step(&s2, state2, x, dt, A2, B2, C2, D2, z2, bias2, 1, y2, nullptr)); }, calls);

    std::printf("{\"m1_step_host_us\": %.3f, \"m2_step_host_us\": %.3f, \"calls\": %d}\n", m1, m2, calls);
    return 0;
}
