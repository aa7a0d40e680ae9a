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
// of 4 when they come first in the list, else 0, ctl[2] = items in runs of 2
// or 4) followed by the items.
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

// Position of item q of an expert's n items in the work list. qbefore and
// rbefore count the items of lower experts in runs of 4 and not; quad_items
// is the number of items in runs of 4 over all experts. With runs_first (when
// the big-cell kernel takes the runs of 4) the items in runs of 4 of every
// expert come first, in ascending expert order, then the remaining items
// (runs of 2 and single items), also by expert; otherwise each expert's items
// are together, in ascending expert order (its runs then sit next to its other
// items, which read the same weights: better for L2 when one kernel takes all).
__host__ __device__ inline int item_slot(int q, int n, int qbefore, int rbefore, int quad_items,
                                         bool runs_first)
{
    if (!runs_first) return qbefore + rbefore + q;
    const int n4 = n & ~3;
    return q < n4 ? qbefore + q : quad_items + rbefore + (q - n4);
}

// Wavefront scans and reductions on DPP lane moves (register to register,
// no LDS round trip): within each row of 16 lanes, Hillis-Steele steps
// row_shr 1, 2, 4, 8; then row_bcast 15 adds row 0's total to row 1 and row
// 2's to row 3, and row_bcast 31 adds lane 31's (rows 0-1) to rows 2 and 3.
// A lane whose source is outside its row, or whose row is masked off, takes
// `id` (the operation's identity). Every lane of the wavefront must be active.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp_move(int v, int id)
{
    return __builtin_amdgcn_update_dpp(id, v, CTRL, ROWS, 0xf, false);
}
enum : int { kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143 };

// inclusive prefix sum across the 64 lanes of a wave
__device__ __forceinline__ int wave_inclusive_scan(int v, int /*lane*/)
{
    v += dpp_move<kRowShr + 1>(v, 0);
    v += dpp_move<kRowShr + 2>(v, 0);
    v += dpp_move<kRowShr + 4>(v, 0);
    v += dpp_move<kRowShr + 8>(v, 0);
    v += dpp_move<kRowBcast15, 0xa>(v, 0);
    v += dpp_move<kRowBcast31, 0xc>(v, 0);
    return v;
}

// sum over the wave (the same value in every lane)
__device__ __forceinline__ int wave_sum(int v)
{
    return __builtin_amdgcn_readlane(wave_inclusive_scan(v, 0), kWave - 1);
}

// maximum over the wave (the same value in every lane)
__device__ __forceinline__ int wave_max(int v)
{
    constexpr int lo = -2147483647 - 1;
    v = max(v, dpp_move<kRowShr + 1>(v, lo));
    v = max(v, dpp_move<kRowShr + 2>(v, lo));
    v = max(v, dpp_move<kRowShr + 4>(v, lo));
    v = max(v, dpp_move<kRowShr + 8>(v, lo));
    v = max(v, dpp_move<kRowBcast15, 0xa>(v, lo));
    v = max(v, dpp_move<kRowBcast31, 0xc>(v, lo));
    return __builtin_amdgcn_readlane(v, kWave - 1);
}

// maximum over the 16 lanes of each DPP row (lanes 16q .. 16q+15): xor-1 and
// xor-2 quad permutes, then the mirrors within 8 and within 16 lanes. Every
// lane of a row must be active (rows may differ).
enum : int { kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140 };
__device__ __forceinline__ int row16_max(int v)
{
    v = max(v, dpp_move<kQuadXor1>(v, v));
    v = max(v, dpp_move<kQuadXor2>(v, v));
    v = max(v, dpp_move<kRowHalfMirror>(v, v));
    v = max(v, dpp_move<kRowMirror>(v, v));
    return v;
}

// Compact expert outputs (moe_forward with 16-bit element types): each row of
// y is cut into blocks of kY16Block columns; a block holds binary16 values s
// and one exponent e (int8) and stands for s * 2^-e exactly. The exponents are
// stored block-major, [block][max_rows], so that a wavefront's 64 rows of one
// block are one contiguous 64-byte store. With M the
// block's largest magnitude (NaN counted as 0), e = 15 - k for M = m * 2^k,
// m in [1/2, 1), clamped to [-112, 100] (0 when M is 0 or infinite), so that
// M * 2^e lies in [2^14, 2^15); s = v * 2^e rounded to binary16, nearest even.
constexpr int kY16Block = 128;

__device__ __forceinline__ int y16_exponent(float M)
{
    if (!(M > 0.0f) || __builtin_isinf(M)) return 0;
    const int e = 15 - __builtin_amdgcn_frexp_expf(M);
    return min(max(e, -112), 100);
}

// maximum over the 16 lanes of each DPP row of non-negative floats (fmax
// ignores NaN, as the block maximum does); every lane of a row must be active
__device__ __forceinline__ float row16_fmax(float v)
{
    v = __builtin_fmaxf(v, __int_as_float(dpp_move<kQuadXor1>(__float_as_int(v), 0)));
    v = __builtin_fmaxf(v, __int_as_float(dpp_move<kQuadXor2>(__float_as_int(v), 0)));
    v = __builtin_fmaxf(v, __int_as_float(dpp_move<kRowHalfMirror>(__float_as_int(v), 0)));
    v = __builtin_fmaxf(v, __int_as_float(dpp_move<kRowMirror>(__float_as_int(v), 0)));
    return v;
}

// 2^e as a float, for e in [-126, 127]: scaling by it is exact (as ldexp)
// wherever the product is a normal number
__device__ __forceinline__ float pow2f(int e) { return __int_as_float((e + 127) << 23); }

// Per-expert output ranges: lane l owns expert `expert` (its value in lane l)
// with n entries. Each lane writes the first kOwnEntries entries of its own
// expert; the rest of a heavy expert's entries are written by the whole
// wavefront, heavy expert after heavy expert, lane q writing entries
// kOwnEntries + q, + 64, ..., so that they are not written by one lane alone.
// Every lane of the wavefront must call these (n = 0 for lanes without an
// expert); the shuffles run with every lane active.
constexpr int kOwnEntries = 8;

// tiles[t0 + j] = expert for j < n
__device__ __forceinline__ void wave_fill_tiles(int t0, int n, int expert, int lane,
                                                int32_t *__restrict__ tiles)
{
    for (int q = 0; q < n && q < kOwnEntries; ++q) tiles[t0 + q] = expert;
    uint64_t heavy = __ballot(n > kOwnEntries);
    while (heavy) {
        const int src = __ffsll((unsigned long long)heavy) - 1;
        heavy &= heavy - 1;
        const int ns = __shfl(n, src), ts = __shfl(t0, src), ex = __shfl(expert, src);
        for (int q = kOwnEntries + lane; q < ns; q += kWave) tiles[ts + q] = ex;
    }
}

// work item q of an expert with n items whose rows are [r0, r0 + rows), at its
// work-list slot; items starting at or past max_rows are dropped and rows are
// cut at max_rows (a plan within its bound reaches neither)
__device__ __forceinline__ void put_item(int q, int n, int r0, int rows, int qbefore, int rbefore,
                                         int quad_items, bool runs_first, int expert,
                                         int max_items, int max_rows, WorkItem *__restrict__ items)
{
    const int idx = item_slot(q, n, qbefore, rbefore, quad_items, runs_first);
    const int row = r0 + q * kItemRows;
    if (idx < max_items && row < max_rows) {
        WorkItem it;
        it.expert = expert;
        it.row0 = row;
        it.nrows = min(min(kItemRows, rows - q * kItemRows), max_rows - row);
        it.run = item_run(q, n);
        items[idx] = it;
    }
}

__device__ __forceinline__ void wave_fill_items(int n, int r0, int rows, int qbefore, int rbefore,
                                                int quad_items, bool runs_first, int expert,
                                                int lane, int max_items, int max_rows,
                                                WorkItem *__restrict__ items)
{
    for (int q = 0; q < n && q < kOwnEntries; ++q)
        put_item(q, n, r0, rows, qbefore, rbefore, quad_items, runs_first, expert, max_items,
                 max_rows, items);
    uint64_t heavy = __ballot(n > kOwnEntries);
    while (heavy) {
        const int src = __ffsll((unsigned long long)heavy) - 1;
        heavy &= heavy - 1;
        const int ns = __shfl(n, src), r0s = __shfl(r0, src), rs = __shfl(rows, src);
        const int qb = __shfl(qbefore, src), rb = __shfl(rbefore, src), ex = __shfl(expert, src);
        for (int q = kOwnEntries + lane; q < ns; q += kWave)
            put_item(q, ns, r0s, rs, qb, rb, quad_items, runs_first, ex, max_items, max_rows,
                     items);
    }
}

// Workgroups of a 1-D grid are dealt to the 8 XCDs round-robin in blockIdx
// order. Give each XCD one contiguous range of the first `nlogical` logical
// block indices (so neighbouring logical blocks share that XCD's L2), with
// the surplus blocks of a host-sized grid at the end of each XCD's queue.
// Returns -1 for a surplus block. bid is the block's index among the blocks
// that take logical blocks (blockIdx.x, or less when the grid puts other
// blocks before them); their number must be a multiple of 8.
__device__ __forceinline__ int xcd_logical_block(int nlogical, int bid)
{
    const int xcd = bid & 7;
    const int local = bid >> 3;
    const int per = (nlogical + 7) >> 3;
    const int lb = xcd * per + local;
    return (local < per && lb < nlogical) ? lb : -1;
}

__device__ __forceinline__ int xcd_logical_block(int nlogical)
{
    return xcd_logical_block(nlogical, blockIdx.x);
}

}  // namespace moe
