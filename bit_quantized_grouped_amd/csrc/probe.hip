// Streaming-read probe: the measured HBM read ceiling that the roofline of
// the weight-streaming kernels is reported against, next to the published
// 8 TB/s.  Each workgroup reads one contiguous 32 KB range with 16-byte
// loads, eight in flight per thread (the configuration that read fastest in
// a sweep of 32-256 KB per workgroup and 1 or 4 loads in flight), and
// writes the XOR of its range to sink[workgroup], so the reads cannot be
// dropped and their result can be checked.
#include "moe_device.h"
#include "moe_launch.h"

namespace moeq4 {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int kProbePieces = kProbeThreads * kProbeUnroll;   // 16-byte pieces per workgroup (32 KB)

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* __restrict__ p,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ sink) {
    __shared__ uint32_t s_x[kProbeThreads / WAVE];
    const size_t base = (size_t)blockIdx.x * kProbePieces;
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
        const size_t i = base + (size_t)u * kProbeThreads + threadIdx.x;
        v[u] = i < n16 ? p[i] : u32x4_t{0, 0, 0, 0};
    }
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
#pragma unroll
    for (int m = WAVE / 2; m >= 1; m /= 2) x ^= shfl_xor(x, m);
    if (threadIdx.x % WAVE == 0) s_x[threadIdx.x / WAVE] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int w = 0; w < kProbeThreads / WAVE; ++w) r ^= s_x[w];
        sink[blockIdx.x] = r;
    }
}

// Launch-latency probe.  Kernel i of a chain reads word i % 2 of buf in every
// workgroup and workgroup 0 writes that value + 1 into word (i + 1) % 2, so
// each launch waits on the previous launch's write through memory, as the two
// launches of a decode token do (h and the chosen experts cross the kernel
// boundary).  With dep = 0 the kernels do nothing: the cost of the launches
// and kernel boundaries alone.
__global__ void launch_probe_kernel(uint32_t* buf, int src, int dep) {
    if (!dep || threadIdx.x != 0) return;
    const uint32_t v = __atomic_load_n(buf + src, __ATOMIC_RELAXED);
    if (blockIdx.x == 0) buf[src ^ 1] = v + 1;
    else if (v == 0xFFFFFFFFu) buf[2] = blockIdx.x;   // keeps every workgroup's read
}

hipError_t launch_launch_probe(uint32_t* buf, int n_launches, int grid_a, int threads_a, int grid_b,
                               int threads_b, int dep, hipStream_t stream) {
    for (int i = 0; i < n_launches; ++i) {
        const bool a = (i & 1) == 0;
        launch_probe_kernel<<<a ? grid_a : grid_b, a ? threads_a : threads_b, 0, stream>>>(buf, i & 1,
                                                                                         dep);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

size_t read_probe_sink_words(size_t bytes) {
    const size_t n16 = bytes / 16;
    return (n16 + kProbePieces - 1) / kProbePieces;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    read_probe_kernel<<<(unsigned)read_probe_sink_words(bytes), kProbeThreads, 0, stream>>>(
        (const u32x4_t*)buf, n16, sink);
    return hipGetLastError();
}

}  // namespace moeq4
