// Routing plan for gfx950: per-block expert histogram, one-workgroup scan
// with the pad-row fill, and a stable placement ranked by wavefront ballots.
//
// Source: "Round 4 Track C: Prefill MoE Plan (mm_clear + mm_hist + mm_scan +
// mm_place) & Epilogue / Gather Audit", section 1, findings 1-3:
//  - the histogram zeroes its own LDS counters and stores every per-block
//    count, so nothing has to clear it beforehand (finding 1);
//  - the scan, one workgroup with one lane per expert, also marks its
//    expert's pad rows -1, which removes the separate clear kernel (finding 1);
//  - the placement rank of an entry is the number of earlier same-expert
//    entries in its block; a serial loop over the block was the bottleneck
//    (finding 2); histogram and scan stay separate launches because one
//    workgroup cannot fill the GPU (finding 3).
// Here the rank comes from ceil(log2 E) wavefront ballots that build each
// lane's equal-expert mask (AMD has no match instruction), a popcount below
// the lane, and a per-(expert, wave) byte table in LDS for the waves before.
// That is exact for any multiplicity, unlike a packed-nibble counter, which
// relies on top-10 routing to bound the count per sub-block.
#include "common.hpp"
#include "launch.hpp"
#include "plan_wave.hpp"

namespace moe {

// bcnt[b][0..E-1]: entries of each expert in block b; bcnt[b][E]: ids == -1;
// bcnt[b][E+1]: other ids outside [0, E). Row stride E+2.
__global__ __launch_bounds__(kPlanBlock) void k_hist(const int32_t *__restrict__ ids, int nent,
                                                     int E, int32_t *__restrict__ bcnt)
{
    __shared__ int h[kMaxExperts + 2];
    const int tid = threadIdx.x;
    for (int e = tid; e < E + 2; e += kPlanBlock) h[e] = 0;
    __syncthreads();
    const int i = blockIdx.x * kPlanBlock + tid;
    if (i < nent) {
        const int e = ids[i];
        const int slot = (e == -1) ? E : ((unsigned)e < (unsigned)E ? e : E + 1);
        atomicAdd(&h[slot], 1);
    }
    __syncthreads();
    int32_t *row = bcnt + (size_t)blockIdx.x * (E + 2);
    for (int e = tid; e < E + 2; e += kPlanBlock) row[e] = h[e];
}

// One workgroup, lane e owns expert e: column scan of bcnt over the blocks
// (boff, cnt), padded rows, exclusive scan over experts (eoff), pad fill,
// tiles and meta.
__global__ __launch_bounds__(kPlanBlock) void k_scan(
    const int32_t *__restrict__ bcnt, int nblk, int E, int K, int tm, int nent,
    int32_t *__restrict__ cnt, int32_t *__restrict__ eoff, int32_t *__restrict__ boff,
    int32_t *__restrict__ tiles, int32_t *__restrict__ stok, float *__restrict__ sw,
    int32_t *__restrict__ meta)
{
    __shared__ int s_sum[16], s_act[16], s_max[16], s_skip[16], s_bad[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int E2 = E + 2;

    int run = 0;
    if (tid < E) {
        int b = 0;
        for (; b + 32 <= nblk; b += 32) {  // 32 independent loads in flight
            int v[32];
#pragma unroll
            for (int q = 0; q < 32; ++q) v[q] = bcnt[(size_t)(b + q) * E2 + tid];
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                boff[(size_t)(b + q) * E + tid] = run;
                run += v[q];
            }
        }
        if (b < nblk) {  // the last < 32 blocks, their loads in flight together too
            int v[32];
#pragma unroll
            for (int q = 0; q < 32; ++q) v[q] = b + q < nblk ? bcnt[(size_t)(b + q) * E2 + tid] : 0;
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                if (b + q < nblk) boff[(size_t)(b + q) * E + tid] = run;
                run += v[q];
            }
        }
    }
    // skipped / bad totals: block-wide sums over the two extra columns
    int skip = 0, bad = 0;
    for (int b = tid; b < nblk; b += kPlanBlock) {
        skip += bcnt[(size_t)b * E2 + E];
        bad += bcnt[(size_t)b * E2 + E + 1];
    }

    const int c = run;
    const int rows = (c + tm - 1) / tm * tm;
    const int incl = wave_inclusive_scan(rows, lane);
    const int act = wave_sum(c > 0 ? 1 : 0);
    const int mx = wave_max(c);
    skip = wave_sum(skip);
    bad = wave_sum(bad);
    if (lane == 63) s_sum[wv] = incl;
    if (lane == 0) {
        s_act[wv] = act;
        s_max[wv] = mx;
        s_skip[wv] = skip;
        s_bad[wv] = bad;
    }
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int v = s_sum[q];
        before += (q < wv) ? v : 0;
        total += v;
    }
    const int start = before + incl - rows;  // exclusive prefix of padded rows

    if (tid < E) {
        cnt[tid] = c;
        eoff[tid] = start;
        for (int r = start + c; r < start + rows; ++r) {  // 0..tm-1 pad rows
            stok[r] = -1;
            sw[r] = 0.0f;
        }
    }
    wave_fill_tiles(start / tm, tid < E ? rows / tm : 0, tid, lane, tiles);
    if (tid == 0) {
        int nact = 0, maxc = 0, nskip = 0, nbad = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            nact += s_act[q];
            maxc = max(maxc, s_max[q]);
            nskip += s_skip[q];
            nbad += s_bad[q];
        }
        eoff[E] = total;
        meta[kMetaNent] = nent;
        meta[kMetaNblk] = nblk;
        meta[kMetaNr] = total;
        meta[kMetaNt] = total / tm;
        meta[kMetaNactive] = nact;
        meta[kMetaMaxcnt] = maxc;
        meta[kMetaNskip] = nskip;
        meta[kMetaNbad] = nbad;
        meta[kMetaTm] = tm;
        meta[kMetaE] = E;
        meta[kMetaK] = K;
    }
}

// sum of the bytes 0..n-1 of a 16-byte value (n in 0..15)
__device__ __forceinline__ int bytes_below(uint4 v, int n)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    int s = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) s += (q < n) ? (int)((w[q >> 2] >> (8 * (q & 3))) & 0xffu) : 0;
    return s;
}

// One workgroup per block of 1024 entries, one entry per lane.
// row(i) = eoff[e] + boff[b][e] + (same-expert entries in earlier waves of
// the block) + (same-expert lanes below this one in the wave).
__global__ __launch_bounds__(kPlanBlock) void k_place(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int nent, int E, int K, int nbits,
    const int32_t *__restrict__ eoff, const int32_t *__restrict__ boff, int32_t *__restrict__ stok,
    float *__restrict__ sw, int32_t *__restrict__ pos)
{
    __shared__ uint4 wc[kMaxExperts];  // byte q of wc[e]: entries of expert e in wave q
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int e = tid; e < E; e += kPlanBlock) wc[e] = make_uint4(0u, 0u, 0u, 0u);

    const int i = blockIdx.x * kPlanBlock + tid;
    const bool inb = i < nent;
    const int e = inb ? ids[i] : -1;
    const bool valid = (unsigned)e < (unsigned)E;

    // lanes holding the same expert: AND over the id bits of (ballot of lanes
    // whose bit is set) or its complement
    uint64_t same = __ballot(valid);
    for (int p = 0; p < nbits; ++p) {
        const bool bit = (e >> p) & 1;
        const uint64_t bl = __ballot(bit);
        same &= bit ? bl : ~bl;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(same & below);
    const int count = __popcll(same);

    __syncthreads();  // wc zeroed
    if (valid && rank == 0) reinterpret_cast<unsigned char *>(wc)[e * 16 + wv] = (unsigned char)count;
    __syncthreads();

    if (valid) {
        const int before = bytes_below(wc[e], wv);
        const int row = eoff[e] + boff[(size_t)blockIdx.x * E + e] + before + rank;
        pos[i] = row;
        stok[row] = i / K;
        sw[row] = w[i];
    } else if (inb) {
        pos[i] = -1;
    }
}

// A workgroup barrier for LDS traffic only: this wavefront's LDS operations
// complete, then s_barrier. __syncthreads()'s release fence would also wait
// for every global store in flight (a memory round trip), which nothing in
// the plan reads back before the kernel ends. As inline asm with a memory
// clobber, so that the compiler moves no LDS access across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited
    asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// Fused plan for up to kFusedMaxBlocks blocks: one launch instead of three.
// Each workgroup (block b of 1024 entries) counts every entry of the layer
// into LDS -- per-expert totals and the counts of the blocks before b -- so it
// knows the padded expert offsets and its own block offsets without waiting
// for the other workgroups; then it places its own entries exactly as k_place
// does. The per-expert layer-wide outputs (cnt, eoff, pad rows, tiles and,
// when asked, the grouped FFN's work items) of expert e are written by
// workgroup e % nblk, so that no workgroup carries them all; the last
// wavefront of workgroup 0 writes eoff[E], meta and the item counts at the
// end, beside the other wavefronts' pad rows. The redundant counting costs
// nblk * nent LDS atomics in total (20 x 20,480 at T=2048, top-10), far less
// than two extra dependent launches. Each lane issues all its loads of ids
// at once (at most kFusedMaxBlocks), and its own entry's id and router
// weight, before it clears the counters, so that neither the counting nor the
// placement waits for more than one load latency. The waves' partial sums are
// combined by wavefront scans on 16 lanes (one LDS read per array).
// One LDS atomic per entry counts it twice: the low 16 bits of s_cnt[e] count
// all entries of expert e, the high 16 bits those before this block (at most
// kFusedMaxBlocks * kPlanBlock = 32,768 entries, so neither half overflows).
constexpr int kFusedMaxBlocks = 32;
static_assert(kFusedMaxBlocks * kPlanBlock <= 65535, "16-bit halves of the fused counters");

__global__ __launch_bounds__(kPlanBlock) void k_plan_fused(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int nent, int E, int K, int tm,
    int nbits, int32_t *__restrict__ cnt, int32_t *__restrict__ eoff, int32_t *__restrict__ boff,
    int32_t *__restrict__ tiles, int32_t *__restrict__ stok, float *__restrict__ sw,
    int32_t *__restrict__ pos, int32_t *__restrict__ meta, int32_t *__restrict__ ctl,
    WorkItem *__restrict__ items, int max_items, int max_rows, int runs_first)
{
    // s_cnt[E]: ids == -1 (skipped entries), s_cnt[E + 1]: other ids outside [0, E)
    __shared__ int s_cnt[kMaxExperts + 2], s_eoff[kMaxExperts];
    __shared__ uint4 wc[kMaxExperts];  // byte q of wc[e]: entries of expert e in wave q
    __shared__ int s_sum[16], s_act[16], s_max[16], s_qsum[16], s_rsum[16], s_psum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int b = blockIdx.x;
    const int bstart = b * kPlanBlock;
    // this lane's own entry (placed in step 3), and the entries it counts:
    // entry tid + u * kPlanBlock for every block u (nent <= U * kPlanBlock),
    // all loads issued before the counters are cleared. A wavefront whose
    // entries of block u all lie past nent skips that load; a lane past nent
    // in a wavefront that loads reads the last entry and does not count it.
    const int i = bstart + tid;
    const bool inb = i < nent;
    const int e = inb ? ids[i] : -1;
    const float wi = inb ? w[i] : 0.0f;
    constexpr int U = kFusedMaxBlocks;
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        v[u] = -1;
        if ((tid & ~(kWave - 1)) + u * kPlanBlock < nent)  // wave-uniform
            v[u] = ids[min(tid + u * kPlanBlock, nent - 1)];
    }
    for (int q = tid; q < E; q += kPlanBlock) {
        s_cnt[q] = 0;
        wc[q] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid < 2) s_cnt[E + tid] = 0;
    lds_barrier();

    // 1. histogram of all entries, and of the entries before this block (ids
    // outside [0, E) into the two counters past the experts')
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = tid + u * kPlanBlock;
        const int ej = v[u];
        if (j < nent)
            atomicAdd(&s_cnt[(unsigned)ej < (unsigned)E ? ej : (ej == -1 ? E : E + 1)],
                      j < bstart ? 0x10001 : 1);
    }
    lds_barrier();

    // 2. padded rows and their exclusive scan over experts (lane e = expert e)
    const int c = tid < E ? s_cnt[tid] & 0xffff : 0;
    const int rows = (c + tm - 1) / tm * tm;
    const int incl = wave_inclusive_scan(rows, lane);
    const int act = wave_sum(c > 0 ? 1 : 0);
    const int mx = wave_max(c);
    // work items of this expert, in runs of 4 and not (only needed by workgroup 0)
    const int nit = (rows + kItemRows - 1) / kItemRows;
    const int nit4 = nit & ~3;
    const int qincl = wave_inclusive_scan(nit4, lane);
    const int rincl = wave_inclusive_scan(nit - nit4, lane);
    const int pairs = wave_sum(nit - nit4 >= 2 ? 2 : 0);  // items in this wave's runs of 2
    if (lane == 63) {
        s_sum[wv] = incl;
        s_qsum[wv] = qincl;
        s_rsum[wv] = rincl;
    }
    if (lane == 0) {
        s_act[wv] = act;
        s_max[wv] = mx;
        s_psum[wv] = pairs;
    }
    lds_barrier();
    // the 16 waves' sums, scanned on lanes 0..15 of every wavefront; wave wv
    // takes the sums of the waves before it from lane wv - 1
    const int ql = lane & 15;
    const int cs = wave_inclusive_scan(lane < 16 ? s_sum[ql] : 0, lane);
    const int cq = wave_inclusive_scan(lane < 16 ? s_qsum[ql] : 0, lane);
    const int cr = wave_inclusive_scan(lane < 16 ? s_rsum[ql] : 0, lane);
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int total = __builtin_amdgcn_readlane(cs, 15);
    const int qtotal = __builtin_amdgcn_readlane(cq, 15);
    const int rtotal = __builtin_amdgcn_readlane(cr, 15);
    const int before = wvu ? __builtin_amdgcn_readlane(cs, wvu - 1) : 0;
    const int qbefore = qincl - nit4 + (wvu ? __builtin_amdgcn_readlane(cq, wvu - 1) : 0);
    const int rbefore = rincl - (nit - nit4) + (wvu ? __builtin_amdgcn_readlane(cr, wvu - 1) : 0);
    const int start = before + incl - rows;
    if (tid < E) {
        s_eoff[tid] = start;
        boff[(size_t)b * E + tid] = s_cnt[tid] >> 16;
    }
    {
        // expert tid's layer-wide outputs, by workgroup tid % nblk
        const bool mine = tid < E && tid % (int)gridDim.x == b;
        if (mine) {  // (its pad rows: after the placement's barrier, below)
            cnt[tid] = c;
            eoff[tid] = start;
        }
        wave_fill_tiles(start / tm, mine ? rows / tm : 0, tid, lane, tiles);
        if (items)  // rows past max_rows (not reached by a plan within its bound) are dropped
            wave_fill_items(mine ? nit : 0, start, rows, qbefore, rbefore, qtotal,
                            runs_first != 0, tid, lane, max_items, max_rows, items);
    }

    // 3. placement of this block's entries (as k_place, offsets from LDS)
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t same = __ballot(valid);
    for (int p = 0; p < nbits; ++p) {
        const bool bit = (e >> p) & 1;
        const uint64_t bl = __ballot(bit);
        same &= bit ? bl : ~bl;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(same & below);
    const int count = __popcll(same);
    if (valid && rank == 0) reinterpret_cast<unsigned char *>(wc)[e * 16 + wv] = (unsigned char)count;
    lds_barrier();
    if (valid) {
        const int row = s_eoff[e] + (s_cnt[e] >> 16) + bytes_below(wc[e], wv) + rank;
        pos[i] = row;
        stok[row] = i / K;
        sw[row] = wi;
    } else if (inb) {
        pos[i] = -1;
    }
    // pad rows (token -1, weight +0) of the experts this workgroup owns
    // (e = b + k nblk): 16 threads per expert write its contiguous pad rows
    const int nblk = gridDim.x;
    const int nown = (E - b + nblk - 1) / nblk;
    for (int k = tid >> 4; k < nown; k += kPlanBlock / 16) {
        const int ex = b + k * nblk;
        const int ce = s_cnt[ex] & 0xffff;
        const int re = (ce + tm - 1) / tm * tm;
        for (int r = ce + (tid & 15); r < re; r += 16) {
            stok[s_eoff[ex] + r] = -1;
            sw[s_eoff[ex] + r] = 0.0f;
        }
    }
    // the layer-wide counts (meta, eoff[E], the work list's item counts), by
    // the last wavefront of workgroup 0, off the placement's critical path
    if (b == 0 && wv == kPlanBlock / kWave - 1) {
        const bool l16 = lane < 16;  // the 16 waves' sums, on 16 lanes
        const int ptotal = wave_sum(l16 ? s_psum[lane & 15] : 0);
        const int nact = wave_sum(l16 ? s_act[lane & 15] : 0);
        const int maxc = wave_max(l16 ? s_max[lane & 15] : 0);
        const int nskip = s_cnt[E] & 0xffff;
        const int nbad = s_cnt[E + 1] & 0xffff;
        if (lane == 0) {
            eoff[E] = total;
            meta[kMetaNent] = nent;
            meta[kMetaNblk] = gridDim.x;
            meta[kMetaNr] = total;
            meta[kMetaNt] = total / tm;
            meta[kMetaNactive] = nact;
            meta[kMetaMaxcnt] = maxc;
            meta[kMetaNskip] = nskip;
            meta[kMetaNbad] = nbad;
            meta[kMetaTm] = tm;
            meta[kMetaE] = E;
            meta[kMetaK] = K;
            if (items) {
                ctl[0] = min(qtotal + rtotal, max_items);
                ctl[1] = runs_first ? min(qtotal, max_items) & ~3 : 0;
                ctl[2] = min(qtotal + ptotal, max_items);
            }
        }
    }
}

// Plan of at most one wavefront of entries (decode-sized calls): the outputs
// of k_plan_fused (with one block) from a single 64-lane workgroup, so that no
// barrier is needed and the launch has one wavefront to start
// (plan_wave_body).
__global__ __launch_bounds__(kWave) void k_plan_wave(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int nent, int E, int K, int tm,
    int nbits, int32_t *__restrict__ cnt, int32_t *__restrict__ eoff, int32_t *__restrict__ boff,
    int32_t *__restrict__ tiles, int32_t *__restrict__ stok, float *__restrict__ sw,
    int32_t *__restrict__ pos, int32_t *__restrict__ meta, int32_t *__restrict__ ctl,
    WorkItem *__restrict__ items, int max_items, int max_rows, int runs_first)
{
    __shared__ int s_cnt[kMaxExperts], s_eoff[kMaxExperts];
    plan_wave_body(ids, w, nent, E, K, tm, nbits, cnt, eoff, boff, tiles, stok, sw, pos, meta, ctl,
                   items, max_items, max_rows, runs_first, s_cnt, s_eoff);
}

int plan_fused_max_blocks() { return kFusedMaxBlocks; }

hipError_t launch_plan_fused(const int32_t *ids, const float *w, int nent, int E, int K, int tm,
                             int nblk, int32_t *cnt, int32_t *eoff, int32_t *boff, int32_t *tiles,
                             int32_t *stok, float *sw, int32_t *pos, int32_t *meta,
                             void *ffn_scratch, int64_t max_items, int64_t max_rows,
                             bool runs_first, hipStream_t s)
{
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    int32_t *ctl = static_cast<int32_t *>(ffn_scratch);
    WorkItem *items = ffn_scratch ? reinterpret_cast<WorkItem *>(static_cast<char *>(ffn_scratch) +
                                                                 kCtlBytes)
                                  : nullptr;
    if (nent <= kWave)  // one wavefront of entries (decode-sized calls)
        hipLaunchKernelGGL(k_plan_wave, dim3(1), dim3(kWave), 0, s, ids, w, nent, E, K, tm, nbits,
                           cnt, eoff, boff, tiles, stok, sw, pos, meta, ctl, items,
                           (int)max_items, (int)max_rows, runs_first ? 1 : 0);
    else
        hipLaunchKernelGGL(k_plan_fused, dim3(nblk), dim3(kPlanBlock), 0, s, ids, w, nent, E, K,
                           tm, nbits, cnt, eoff, boff, tiles, stok, sw, pos, meta, ctl, items,
                           (int)max_items, (int)max_rows, runs_first ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_hist(const int32_t *ids, int nent, int E, int nblk, int32_t *bcnt, hipStream_t s)
{
    hipLaunchKernelGGL(k_hist, dim3(nblk), dim3(kPlanBlock), 0, s, ids, nent, E, bcnt);
    return hipGetLastError();
}

hipError_t launch_scan(const int32_t *bcnt, int nblk, int E, int K, int tm, int nent, int32_t *cnt,
                       int32_t *eoff, int32_t *boff, int32_t *tiles, int32_t *stok, float *sw,
                       int32_t *meta, hipStream_t s)
{
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kPlanBlock), 0, s, bcnt, nblk, E, K, tm, nent, cnt,
                       eoff, boff, tiles, stok, sw, meta);
    return hipGetLastError();
}

hipError_t launch_place(const int32_t *ids, const float *w, int nent, int E, int K, int nblk,
                        const int32_t *eoff, const int32_t *boff, int32_t *stok, float *sw,
                        int32_t *pos, hipStream_t s)
{
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    hipLaunchKernelGGL(k_place, dim3(nblk), dim3(kPlanBlock), 0, s, ids, w, nent, E, K, nbits, eoff,
                       boff, stok, sw, pos);
    return hipGetLastError();
}

}  // namespace moe
