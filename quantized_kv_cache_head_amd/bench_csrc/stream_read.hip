// stream_read.hip -- read-only streaming kernel that calibrates the HBM
// roofline of the benchmark: how fast one launch can read a buffer of a given
// size with 16-byte vector loads on this part.  Not part of libkvq: built into
// libkvq_bench.so and loaded by bench.py only.
//
// Each workgroup of 256 threads reads one contiguous chunk of the buffer, U
// loads of 16 bytes in flight per thread, and folds the words into a value
// that is stored only if it matches an impossible constant (so the loads
// cannot be dropped).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

template <int U>
__global__ __launch_bounds__(256) void stream_read(const u32x4_t* __restrict__ p, uint64_t n16, uint32_t* sink) {
    gptr<u32x4_t> g = (gptr<u32x4_t>)p;
    const uint64_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t b0 = (uint64_t)blockIdx.x * chunk;
    const uint64_t b1 = b0 + chunk < n16 ? b0 + chunk : n16;
    uint32_t acc = 0;
    for (uint64_t i = b0 + threadIdx.x; i < b1; i += 256ull * U) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t j = i + 256ull * u;
            v[u] = g[j < b1 ? j : b1 - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16) starting at `buf` with `grid` workgroups on
// `stream` (a hipStream_t; NULL = the null stream).  `sink` is a device
// buffer of at least `grid` uint32 that is written only in an impossible case.
// Returns 0, or the hipError_t of the launch.
extern "C" __attribute__((visibility("default"))) int kvq_bench_stream_read(const void* buf, uint64_t bytes,
                                                                              int grid, uint32_t* sink,
                                                                              void* stream) {
    if (!buf || !sink || grid < 1 || bytes < 16 || bytes % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read<8>, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const u32x4_t*>(buf), bytes / 16, sink);
    return (int)hipGetLastError();
}
