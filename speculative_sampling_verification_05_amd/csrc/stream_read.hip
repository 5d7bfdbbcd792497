// stream_read.hip - a plain streaming read of a device buffer, the practical
// HBM read ceiling that the verification kernels' statistics stream is
// measured against. Measurement only: nothing on the verification path calls
// it. Same access pattern as the statistics stream: each wavefront reads a
// contiguous range of 1 KiB chunks (64 lanes x 16 bytes) with 16-byte
// non-temporal loads, two groups of four loads in flight; the words are
// folded by XOR and one word per wavefront is stored only if the fold hits a
// value chosen by the caller, so the loads cannot be dropped.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;
constexpr int kGroup = 4;

template <int CPW>
__global__ __launch_bounds__(256) void k_read(const u32x4* p, int64_t n16, uint32_t key, uint32_t* sink) {
    const int lane = static_cast<int>(threadIdx.x & (kWave - 1));
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
    const int64_t c0 = wave * CPW;
    u32x4 acc = {0u, 0u, 0u, 0u};
    u32x4 a[kGroup], b[kGroup];
    auto load = [&](u32x4* q, int g) {
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const int64_t i = (c0 + g * kGroup + u) * kWave + lane;
            q[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto eat = [&](const u32x4* q) {
#pragma unroll
        for (int u = 0; u < kGroup; ++u) acc ^= q[u];
    };
    constexpr int NG = CPW / kGroup;
    load(a, 0);
#pragma unroll
    for (int g = 1; g < NG; g += 2) {
        load(b, g);
        eat(a);
        if (g + 1 < NG) load(a, g + 1);
        eat(b);
    }
    if (NG % 2 == 1) eat(a);
    const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == key) sink[wave] = f;
}

template <int CPW>
void launch(const void* p, int64_t bytes, uint32_t key, uint32_t* sink, hipStream_t st, hipEvent_t e0,
            hipEvent_t e1) {
    const int64_t n16 = bytes / 16;
    const int64_t waves = (n16 + int64_t(CPW) * kWave - 1) / (int64_t(CPW) * kWave);
    const int64_t blocks = (waves + 3) / 4;
    hipExtLaunchKernelGGL((k_read<CPW>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, e0, e1, 0,
                          static_cast<const u32x4*>(p), n16, key, sink);
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) from device pointer p with
// `cpw` chunks per wavefront (8, 16, 24, 32 or 64); sink must hold one word per
// wavefront. Events (hipEvent_t, may be NULL) are bound to the dispatch.
// Returns 0, or -1 for bad arguments, -3 if the launch failed.
int stream_read(const void* p, int64_t bytes, int32_t cpw, uint32_t key, uint32_t* sink, void* stream, void* e0,
                void* e1) {
    if (!p || !sink || bytes < 16 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15u) != 0) return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipEvent_t a = static_cast<hipEvent_t>(e0), b = static_cast<hipEvent_t>(e1);
    switch (cpw) {
        case 8: launch<8>(p, bytes, key, sink, st, a, b); break;
        case 16: launch<16>(p, bytes, key, sink, st, a, b); break;
        case 24: launch<24>(p, bytes, key, sink, st, a, b); break;
        case 32: launch<32>(p, bytes, key, sink, st, a, b); break;
        case 64: launch<64>(p, bytes, key, sink, st, a, b); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Wavefronts (sink words) a call with these arguments uses.
int64_t stream_read_waves(int64_t bytes, int32_t cpw) {
    if (cpw < 1) return -1;
    const int64_t n16 = bytes / 16;
    return (n16 + int64_t(cpw) * kWave - 1) / (int64_t(cpw) * kWave) + 3;
}

}  // extern "C"
