// Streaming-read reference: a measurement aid for the HBM-bound kernels'
// rooflines, not a step of the method.  The rate at which this kernel reads a
// large buffer is what a plain read can get from this GPU's HBM, the measured
// denominator beside the 8 TB/s of the data sheet.
//
// Every 16-byte piece of the buffer is read once, with a non-temporal load, in
// a grid-stride walk (consecutive lanes read consecutive pieces; each lane keeps
// kUnroll loads in flight).  The grid gives each thread at most 64 pieces
// and the launch at least 2,048 workgroups of 256 threads, up to one sink word
// per wave (32,768 workgroups): over 8 GiB that is 32,768, the fastest of the
// shapes measured (7.0 TB/s, against 6.5 with 2,048 workgroups and 6.8 with
// 8,192), and a buffer of a few MB gets 2,048, which reads it in one round
// instead of waiting on the dispatch of mostly idle workgroups.  The words
// a wave read are folded with XOR into one word that the wave's first lane
// writes to the sink, so no load is dead and the XOR of all sink words equals
// the XOR of every 32-bit word of the buffer.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace minikv {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 8;

__device__ __forceinline__ uint32_t fold(const u32x4& v) { return (v[0] ^ v[1]) ^ (v[2] ^ v[3]); }

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                  uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
    }
    for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(src + i));
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, kWave);
    if (threadIdx.x % kWave == 0) sink[blockIdx.x * (kProbeThreads / kWave) + threadIdx.x / kWave] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int sink_words, hipStream_t stream) {
    constexpr size_t kPiecesPerThread = 64;
    const size_t n16 = bytes / 16;
    const size_t max_blocks = (size_t)sink_words / (kProbeThreads / kWave);
    const size_t want = (n16 + kProbeThreads * kPiecesPerThread - 1) / (kProbeThreads * kPiecesPerThread);
    const int blocks = (int)std::min(max_blocks, std::max<size_t>(2048, want));
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4*>(src), n16, sink);
    return hipGetLastError();
}

}  // namespace minikv
