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

// non-temporal accesses for data touched once here (the expert outputs read
// by the combine, the layer output). The gather's destination rows are
// stored with cache policy sc1 instead (below).
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
// A token's row is copied to up to K rows, in no particular order of r. To
// fetch each token row into one L2 only, row r is copied by the XCD
// (stok[r] mod 8) of its token (a pad row by r mod 8): workgroup b scans the
// kGatherWaves x 64 rows of row group b / 8 and copies those owned by
// XCD b mod 8 (the hardware deals the workgroups of a 1-D grid to the 8 XCDs
// round robin). Each row has exactly one owner whatever the placement; only
// the L2 reuse depends on it. A wavefront copies its matching rows
// kGatherBatch at a time, with kGatherVec loads per lane and row in flight.
// Small workgroups, one row at a time and 5 vectors per lane (a whole
// 5,120-byte row per pass at the prefill shape) measured fastest: prefill
// gather 29.4 us with 4 wavefronts, 4 rows and 4 vectors; 25.4 with 4, 2, 5;
// 24.2 with 2, 1, 5 (more workgroups in flight, fewer registers each). The
// rows are stored with cache policy sc1 through a descriptor over the row:
// 21.4 us, against 24.1 with default-policy stores and 26.7 non-temporal.
constexpr int kGatherStorePolicy = 16;  // sc1
constexpr int kGatherWaves = 2;
constexpr int kGatherBatch = 1;
constexpr int kGatherVec = 5;

__global__ __launch_bounds__(kGatherWaves * kWave) void k_gather(
    const uint4 *__restrict__ x, int T, int vpr, const int32_t *__restrict__ stok,
    const int32_t *__restrict__ meta, int64_t max_rows, uint4 *__restrict__ xs)
{
    const int xcd = blockIdx.x & 7;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t r0 = ((int64_t)(blockIdx.x >> 3) * kGatherWaves + wave) * kWave;
    const int64_t nr = min((int64_t)meta[kMetaNr], max_rows);
    if (r0 >= nr) return;
    const int lane = threadIdx.x & 63;
    const int64_t r = r0 + lane;
    const int t = r < nr ? stok[r] : -1;
    const int owner = (unsigned)t < (unsigned)T ? (t & 7) : (int)(r & 7);
    uint64_t mine = __ballot(r < nr && owner == xcd);
    while (mine) {
        int64_t rr[kGatherBatch];  // -1: empty slot of the batch
        int tt[kGatherBatch];
#pragma unroll
        for (int u = 0; u < kGatherBatch; ++u) {
            rr[u] = -1;
            tt[u] = -1;
            if (mine) {
                const int src = __ffsll((unsigned long long)mine) - 1;
                mine &= mine - 1;
                rr[u] = r0 + src;
                tt[u] = __builtin_amdgcn_readlane(t, src);
            }
        }
        for (int j0 = lane; j0 < vpr; j0 += kGatherVec * kWave) {
            uint4 v[kGatherBatch][kGatherVec];
#pragma unroll
            for (int u = 0; u < kGatherBatch; ++u)
#pragma unroll
                for (int q = 0; q < kGatherVec; ++q) {
                    const int j = j0 + q * kWave;
                    v[u][q] = (j < vpr && (unsigned)tt[u] < (unsigned)T)
                                  ? x[(int64_t)tt[u] * vpr + j]
                                  : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
            for (int u = 0; u < kGatherBatch; ++u)
#pragma unroll
                for (int q = 0; q < kGatherVec; ++q) {
                    const int j = j0 + q * kWave;
                    if (j < vpr && rr[u] >= 0) {
                        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
                        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
                            static_cast<void *>(xs + rr[u] * vpr), (short)0, vpr * 16, 0x00020000);
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u4{v[u][q].x, v[u][q].y, v[u][q].z, v[u][q].w}, rd, j * 16, 0,
                            kGatherStorePolicy);
                    }
                }
        }
    }
}

// out[t] = (((+0 + y[pos[tK]]) + y[pos[tK+1]]) + ...) in fp32, k ascending,
// pos < 0 or >= max_rows skipped. One workgroup per token, sized to cover a
// whole row (up to 1024 lanes); a lane takes 4 columns of fp32 rows, or 8
// columns of compact rows (Y16: binary16 values, and the exponent e of their
// 128-column block, block-major: yexp[b * max_rows + row]; each value decoded
// exactly as s * 2^-e). For a lane's
// columns, the rows of up to G entries are loaded first -- every load issued,
// a skipped entry reading row 0 and adding nothing -- then added in k order,
// so one memory latency covers a group. G is instantiated for 2, 4, 8, 10, 12
// and 16 and chosen per launch as the smallest that covers min(K, 16): with a
// fixed G = 16, top-10 lanes loaded 6 rows for nothing (prefill combine 26.9
// -> 23.0 us, micro-batch 13.6 -> 11.2, decode 6.8 -> 6.1). (Branching around
// the loads of skipped entries instead, which are the same for every lane of
// the workgroup: prefill 26.9 us, decode 8.0 us; not kept.)
constexpr int kCombineGroup = 16;

template <bool Y16, int G>
__global__ __launch_bounds__(1024) void k_combine(const void *__restrict__ y,
                                                 const int8_t *__restrict__ yexp,
                                                 int64_t max_rows, int d,
                                                 const int32_t *__restrict__ pos, int T, int K,
                                                 float4 *__restrict__ out)
{
    constexpr int COLS = Y16 ? 8 : 4;  // columns per lane
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const int t = blockIdx.x;
    const int32_t *p = pos + (int64_t)t * K;
    const int nvec = d / COLS;
    for (int j = threadIdx.x; j < nvec; j += blockDim.x) {
        float acc[COLS];
#pragma unroll
        for (int c = 0; c < COLS; ++c) acc[c] = 0.f;
        for (int k0 = 0; k0 < K; k0 += G) {
            const int n = min(G, K - k0);
            int row[G];
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int r = u < n ? p[k0 + u] : -1;  // wave-uniform: scalar loads
                row[u] = (r >= 0 && r < max_rows) ? r : -1;
            }
            u4 raw[G];
            int e[G];
#pragma unroll
            for (int u = 0; u < G; ++u) {
                const int64_t r = row[u] >= 0 ? row[u] : 0;
                raw[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u4 *>(y) + r * nvec + j);
                e[u] = Y16 ? -(int)yexp[(int64_t)((j * COLS) / kY16Block) * max_rows + r] : 0;
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
                if (row[u] < 0) continue;  // wave-uniform
                // the loaded words as plain values (a bit cast takes values, not
                // vector elements)
                const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
                if constexpr (Y16) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const uint16_t hbits = (uint16_t)(w[c >> 1] >> (16 * (c & 1)));
                        acc[c] += __builtin_amdgcn_ldexpf((float)__builtin_bit_cast(_Float16, hbits),
                                                          e[u]);
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[c] += __builtin_bit_cast(float, w[c]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < COLS; c += 4)
            store_nt(out + (int64_t)t * (d / 4) + j * (COLS / 4) + c / 4,
                     make_float4(acc[c], acc[c + 1], acc[c + 2], acc[c + 3]));
    }
}

// the smallest group size of the instantiated ones that covers min(K, 16)
// entries, so that no lane loads rows for slots past K
template <bool Y16>
void combine_any(int K, dim3 grid, dim3 block, hipStream_t s, const void *y, const int8_t *yexp,
                 int64_t max_rows, int d, const int32_t *pos, int T, float4 *out)
{
    const int g = K < kCombineGroup ? K : kCombineGroup;
#define MOE_COMBINE(G)                                                                         \
    hipLaunchKernelGGL((k_combine<Y16, G>), grid, block, 0, s, y, yexp, max_rows, d, pos, T, K, \
                       out)
    if (g <= 2)
        MOE_COMBINE(2);
    else if (g <= 4)
        MOE_COMBINE(4);
    else if (g <= 8)
        MOE_COMBINE(8);
    else if (g <= 10)
        MOE_COMBINE(10);
    else if (g <= 12)
        MOE_COMBINE(12);
    else
        MOE_COMBINE(kCombineGroup);
#undef MOE_COMBINE
}

hipError_t launch_gather(const void *x, int elem_bytes, int T, int d, const int32_t *stok,
                         const int32_t *meta, int64_t max_rows, void *xs, hipStream_t s)
{
    const int vpr = d * elem_bytes / 16;
    constexpr int rows_per_group = kGatherWaves * kWave;
    const int64_t blocks = (max_rows + rows_per_group - 1) / rows_per_group * 8;
    hipLaunchKernelGGL(k_gather, dim3((unsigned)blocks), dim3(kGatherWaves * kWave), 0, s,
                       static_cast<const uint4 *>(x), T, vpr, stok, meta, max_rows,
                       static_cast<uint4 *>(xs));
    return hipGetLastError();
}

hipError_t launch_combine(const float *y, int64_t max_rows, const int32_t *pos, int T, int K,
                          int d, float *out, hipStream_t s)
{
    const int threads = min(1024, (d / 4 + kWave - 1) / kWave * kWave);
    combine_any<false>(K, dim3(T), dim3(threads), s, y, nullptr, max_rows, d, pos, T,
                       reinterpret_cast<float4 *>(out));
    return hipGetLastError();
}

hipError_t launch_combine_y16(const uint16_t *y16, const int8_t *yexp, int64_t max_rows,
                              const int32_t *pos, int T, int K, int d, float *out, hipStream_t s)
{
    const int threads = min(1024, (d / 8 + kWave - 1) / kWave * kWave);
    combine_any<true>(K, dim3(T), dim3(threads), s, y16, yexp, max_rows, d, pos, T,
                      reinterpret_cast<float4 *>(out));
    return hipGetLastError();
}

}  // namespace moe
