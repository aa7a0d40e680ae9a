// Streaming-read probe of the benchmark (measurement only; not part of the
// layer's library or its C ABI): reads a device buffer once with 16-byte
// non-temporal loads, the access pattern of the grouped GEMMs' weight streams,
// so that the benchmark can quote in the same run the read rate the GPU
// attains next to the layer's kernels. Built by bench.build_probe() into
// libbench_probe.so beside bench.py.
//
// Each workgroup streams one contiguous chunk: 256 threads x 16 bytes = 4 KB
// per row, 8 rows in flight per thread. (Measured on MI355X: this reaches
// 7.0-7.1 TB/s; a grid-stride walk over the whole buffer stays near 6 TB/s.)
// Every loaded word feeds an XOR that decides a store, so no load can be
// removed.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const uint4 *__restrict__ src,
                                                               size_t n16,
                                                               uint32_t *__restrict__ sink)
{
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const size_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * chunk;
    const size_t b1 = b0 + chunk < n16 ? b0 + chunk : n16;
    size_t i = b0 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < b1; i += kProbeUnroll * kProbeThreads) {
        u4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = __builtin_nontemporal_load(
                reinterpret_cast<const u4 *>(src + i + u * kProbeThreads));
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < b1; i += kProbeThreads) {
        const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(src + i));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // a data-dependent store keeps every load live; it fires only for one
    // checksum value out of 2^32
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

// One streaming read of src (bytes / 16 16-byte words) on `stream`. sink
// [sink_words] receives at most one word per workgroup, and only for one
// checksum value in 2^32; its contents carry no meaning. Returns 0, 1 for a
// bad argument (misaligned src or sink, bytes < 16, sink_words < 1), 3 when
// the launch fails.
extern "C" int bench_stream_read(const void *src, size_t bytes, uint32_t *sink, int sink_words,
                                 void *stream)
{
    if (!src || !sink || reinterpret_cast<uintptr_t>(src) % 16 ||
        reinterpret_cast<uintptr_t>(sink) % 4 || bytes < 16 || sink_words < 1)
        return 1;
    // 32 workgroups per CU on 256 CUs, capped by the sink (one word per workgroup)
    const int blocks = sink_words < 8192 ? sink_words : 8192;
    hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(src),
                       bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
