// Activation gather and fixed-order combine for gfx950. Both are HBM-bound
// copies/reductions: one wavefront per row, 16-byte (dwordx4) accesses.
//
// Gather source: "Round 4 Track C: Prefill MoE Plan ... & Epilogue / Gather
// Audit", section 1, finding 4 -- the routed rows are copied from the
// half-precision activation with wide vector loads and stores, bit for bit.
// Combine source: "Batched resident MoE experts on Apple Silicon: a flat
// parallel expert pass", section 3 -- a fixed per-token top-k summation order
// keeps the result bit-identical from run to run.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kRowsPerBlock = 4;  // one wave per row, 4 waves per workgroup

// non-temporal accesses for data touched once here (the destination rows of
// the gather, the expert outputs read by the combine, the layer output)
__device__ __forceinline__ void store_nt(uint4 *p, uint4 v)
{
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u4{v.x, v.y, v.z, v.w}, reinterpret_cast<u4 *>(p));
}
__device__ __forceinline__ void store_nt(float4 *p, float4 v)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f4{v.x, v.y, v.z, v.w}, reinterpret_cast<f4 *>(p));
}
__device__ __forceinline__ float4 load_nt(const float4 *p)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// xs[r] = x[stok[r]] (bit copy) for r < min(meta[NR], max_rows); zeros on pad
// rows. vpr = 16-byte vectors per row.
__global__ __launch_bounds__(256) void k_gather(const uint4 *__restrict__ x, int T, int vpr,
                                                const int32_t *__restrict__ stok,
                                                const int32_t *__restrict__ meta, int64_t max_rows,
                                                uint4 *__restrict__ xs)
{
    const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    const int64_t nr = min((int64_t)meta[kMetaNr], max_rows);
    if (r >= nr) return;
    const int lane = threadIdx.x & 63;
    const int t = stok[r];
    uint4 *dst = xs + r * vpr;
    if ((unsigned)t < (unsigned)T) {
        const uint4 *src = x + (int64_t)t * vpr;
        int j = lane;
        for (; j + 3 * kWave < vpr; j += 4 * kWave) {  // 4 loads in flight per lane
            const uint4 a = src[j], b = src[j + kWave], c = src[j + 2 * kWave],
                        d = src[j + 3 * kWave];
            store_nt(dst + j, a);
            store_nt(dst + j + kWave, b);
            store_nt(dst + j + 2 * kWave, c);
            store_nt(dst + j + 3 * kWave, d);
        }
        for (; j < vpr; j += kWave) store_nt(dst + j, src[j]);
    } else {
        for (int j = lane; j < vpr; j += kWave) store_nt(dst + j, make_uint4(0u, 0u, 0u, 0u));
    }
}

// out[t] = (((+0 + y[pos[tK]]) + y[pos[tK+1]]) + ...) in fp32, k ascending,
// pos < 0 or >= max_rows skipped. One workgroup per token, sized to cover a
// whole row (one float4 column per lane up to 1024 lanes); for a column, the
// rows of up to kCombineGroup entries are loaded first (independent loads, all
// in flight), then added in k order, so one memory latency covers a group.
constexpr int kCombineGroup = 16;

__global__ __launch_bounds__(1024) void k_combine(const float4 *__restrict__ y, int64_t max_rows,
                                                 int vpr, const int32_t *__restrict__ pos, int T,
                                                 int K, float4 *__restrict__ out)
{
    const int t = blockIdx.x;
    const int32_t *p = pos + (int64_t)t * K;
    for (int j = threadIdx.x; j < vpr; j += blockDim.x) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k0 = 0; k0 < K; k0 += kCombineGroup) {
            const int n = min(kCombineGroup, K - k0);
            int row[kCombineGroup];
#pragma unroll
            for (int u = 0; u < kCombineGroup; ++u) {
                const int r = u < n ? p[k0 + u] : -1;  // wave-uniform: scalar loads
                row[u] = (r >= 0 && r < max_rows) ? r : -1;
            }
            float4 v[kCombineGroup];
#pragma unroll
            for (int u = 0; u < kCombineGroup; ++u)
                v[u] = row[u] >= 0 ? load_nt(y + (int64_t)row[u] * vpr + j)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < kCombineGroup; ++u)
                if (row[u] >= 0) {
                    acc.x += v[u].x;
                    acc.y += v[u].y;
                    acc.z += v[u].z;
                    acc.w += v[u].w;
                }
        }
        store_nt(out + (int64_t)t * vpr + j, acc);
    }
}

hipError_t launch_gather(const void *x, int elem_bytes, int T, int d, const int32_t *stok,
                         const int32_t *meta, int64_t max_rows, void *xs, hipStream_t s)
{
    const int vpr = d * elem_bytes / 16;
    const int64_t blocks = (max_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(k_gather, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint4 *>(x), T, vpr, stok, meta, max_rows,
                       static_cast<uint4 *>(xs));
    return hipGetLastError();
}

hipError_t launch_combine(const float *y, int64_t max_rows, const int32_t *pos, int T, int K,
                          int d, float *out, hipStream_t s)
{
    const int vpr = d / 4;
    const int threads = min(1024, (vpr + kWave - 1) / kWave * kWave);
    hipLaunchKernelGGL(k_combine, dim3(T), dim3(threads), 0, s,
                       reinterpret_cast<const float4 *>(y), max_rows, vpr, pos, T, K,
                       reinterpret_cast<float4 *>(out));
    return hipGetLastError();
}

}  // namespace moe
