// Device-side definitions shared by the gfx950 kernels of the routed MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kPlanBlock = 1024;     // entries per plan block, one per thread
constexpr int kMaxExperts = 1024;    // LDS counters per plan block

// meta[] fields (values fixed by the public header's enum moe_meta_field)
enum : int {
    kMetaNent = 0, kMetaNblk, kMetaNr, kMetaNt, kMetaNactive, kMetaMaxcnt, kMetaNskip,
    kMetaNbad, kMetaTm, kMetaE, kMetaK, kMetaN
};

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// The grouped FFN works on items of at most kItemRows rows of one expert; its
// scratch holds ctl (first kCtlBytes: ctl[0] = items, ctl[1] = items in runs
// of 4) followed by the items.
constexpr int kItemRows = 64;
constexpr size_t kCtlBytes = 256;

// A work item of the grouped FFN: one expert's run of at most kItemRows rows.
// `run` groups consecutive items of one expert whose workgroups share the
// expert's weight tile: run length (1, 2 or 4) | (index in the run << 8).
struct WorkItem {
    int32_t expert;
    int32_t row0;
    int32_t nrows;
    int32_t run;
};

// Run of item q of an expert's n items: runs of 4 first, then one run of 2 if
// at least 2 items remain, else single items. (Completing a last partial run
// of 4 with empty items instead was measured slower on the long prompt in
// chunks and no faster in one call.)
__host__ __device__ inline int32_t item_run(int q, int n)
{
    const int n4 = n & ~3;
    if (q < n4) return 4 | ((q & 3) << 8);
    const int q2 = q - n4;
    if (n - n4 >= 2 && q2 < 2) return 2 | (q2 << 8);
    return 1;
}

// Position of item q of an expert's n items in the work list. The items in
// runs of 4 of every expert come first, in ascending expert order, then the
// remaining items (runs of 2 and single items), also by expert. qbefore and
// rbefore count the items of lower experts in each part; quad_items is the
// number of items in runs of 4 over all experts.
__host__ __device__ inline int item_slot(int q, int n, int qbefore, int rbefore, int quad_items)
{
    const int n4 = n & ~3;
    return q < n4 ? qbefore + q : quad_items + rbefore + (q - n4);
}

__device__ __forceinline__ int wave_sum(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_max(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

// inclusive prefix sum across the 64 lanes of a wave
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    return v;
}

// Workgroups of a 1-D grid are dealt to the 8 XCDs round-robin in blockIdx
// order. Give each XCD one contiguous range of the first `nlogical` logical
// block indices (so neighbouring logical blocks share that XCD's L2), with
// the surplus blocks of a host-sized grid at the end of each XCD's queue.
// Returns -1 for a surplus block. gridDim.x must be a multiple of 8.
__device__ __forceinline__ int xcd_logical_block(int nlogical)
{
    const int xcd = blockIdx.x & 7;
    const int local = blockIdx.x >> 3;
    const int per = (nlogical + 7) >> 3;
    const int lb = xcd * per + local;
    return (local < per && lb < nlogical) ? lb : -1;
}

}  // namespace moe
