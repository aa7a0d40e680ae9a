// The routing plan of a call of at most one wavefront of entries (T*K <= 64,
// decode-sized), computed by one wavefront with no barrier: shared by the
// plan's own one-wavefront launch and by the gate/up launch that plans such a
// call itself (see wave_plan_item).
//
// Source: "Round 4 Track C: Prefill MoE Plan (mm_clear + mm_hist + mm_scan +
// mm_place) & Epilogue / Gather Audit", section 1 (the plan's outputs and
// their ordering); "Batched resident MoE experts on Apple Silicon", section 1
// (the flat job list of a decode step).
#pragma once

#include "common.hpp"

namespace moe {

// experts per lane at most (E <= kMaxExperts)
constexpr int kWaveExperts = kMaxExperts / kWave;

// The outputs of the one-launch plan (one block) for nent <= 64 entries, from
// one wavefront (lane l = entry l and experts [l * epl, (l + 1) * epl), epl =
// ceil(E / 64) <= 16). The ranks come from ceil(log2 E) ballots; the first
// lane of each expert writes its count to s_cnt; each lane then takes its
// experts' counts in order (a running sum plus a wavefront scan for the
// padded-row offsets and the work-list slots) and writes their outputs.
// s_cnt and s_eoff are LDS arrays of kMaxExperts ints owned by the wavefront.
__device__ __forceinline__ void plan_wave_body(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int nent, int E, int K, int tm,
    int nbits, int32_t *__restrict__ cnt, int32_t *__restrict__ eoff, int32_t *__restrict__ boff,
    int32_t *__restrict__ tiles, int32_t *__restrict__ stok, float *__restrict__ sw,
    int32_t *__restrict__ pos, int32_t *__restrict__ meta, int32_t *__restrict__ ctl,
    WorkItem *__restrict__ items, int max_items, int max_rows, int runs_first, int *s_cnt,
    int *s_eoff)
{
    const int lane = threadIdx.x & (kWave - 1);
    const bool inb = lane < nent;
    const int e = inb ? ids[lane] : -1;
    const float wi = inb ? w[lane] : 0.0f;
    const int epl = (E + kWave - 1) / kWave;
    const int e0 = lane * epl;
#pragma unroll
    for (int j = 0; j < kWaveExperts; ++j)
        if (j < epl && e0 + j < E) s_cnt[e0 + j] = 0;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t same = __ballot(valid);
    for (int p = 0; p < nbits; ++p) {
        const bool bit = (e >> p) & 1;
        const uint64_t bl = __ballot(bit);
        same &= bit ? bl : ~bl;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(same & below);
    const int nskip = __popcll(__ballot(inb && e == -1));
    const int nbad = __popcll(__ballot(inb && e != -1 && !valid));
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the counters cleared (lgkmcnt(0))
    if (valid && rank == 0) s_cnt[e] = __popcll(same);
    __builtin_amdgcn_s_waitcnt(0xc07f);

    // this lane's experts: counts, padded rows and items, then the offsets
    int c[kWaveExperts];
    int lrows = 0, lq = 0, lr = 0, lp = 0, lact = 0, lmax = 0;
#pragma unroll
    for (int j = 0; j < kWaveExperts; ++j) {
        c[j] = (j < epl && e0 + j < E) ? s_cnt[e0 + j] : 0;
        const int rows = (c[j] + tm - 1) / tm * tm;
        const int nit = (rows + kItemRows - 1) / kItemRows, nit4 = nit & ~3;
        lrows += rows;
        lq += nit4;
        lr += nit - nit4;
        lp += nit - nit4 >= 2 ? 2 : 0;
        lact += c[j] > 0 ? 1 : 0;
        lmax = max(lmax, c[j]);
    }
    const int srow = wave_inclusive_scan(lrows, lane);
    const int sq = wave_inclusive_scan(lq, lane);
    const int sr = wave_inclusive_scan(lr, lane);
    const int total = __builtin_amdgcn_readlane(srow, kWave - 1);
    const int qtotal = __builtin_amdgcn_readlane(sq, kWave - 1);
    const int rtotal = __builtin_amdgcn_readlane(sr, kWave - 1);
    const int ptotal = wave_sum(lp), nact = wave_sum(lact), maxc = wave_max(lmax);
    int start = srow - lrows, qb = sq - lq, rb = sr - lr;
#pragma unroll
    for (int j = 0; j < kWaveExperts; ++j) {
        const int ex = e0 + j;
        if (!(j < epl && ex < E)) continue;
        const int rows = (c[j] + tm - 1) / tm * tm;
        const int nit = (rows + kItemRows - 1) / kItemRows, nit4 = nit & ~3;
        s_eoff[ex] = start;
        cnt[ex] = c[j];
        eoff[ex] = start;
        boff[ex] = 0;  // one block: no entries before it
        for (int t = 0; t < rows / tm; ++t) tiles[start / tm + t] = ex;
        for (int r = start + c[j]; r < start + rows; ++r) {  // pad rows
            stok[r] = -1;
            sw[r] = 0.0f;
        }
        if (items)
            for (int q = 0; q < nit; ++q)
                put_item(q, nit, start, rows, qb, rb, qtotal, runs_first != 0, ex, max_items,
                         max_rows, items);
        start += rows;
        qb += nit4;
        rb += nit - nit4;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // s_eoff written

    // placement: the expert's offset plus the rank among its lanes
    if (valid) {
        const int row = s_eoff[e] + rank;
        pos[lane] = row;
        stok[row] = lane / K;
        sw[row] = wi;
    } else if (inb) {
        pos[lane] = -1;
    }
    if (lane == 0) {
        eoff[E] = total;
        meta[kMetaNent] = nent;
        meta[kMetaNblk] = 1;
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

// The work item of logical block lb of a gate/up launch over the plan that
// plan_wave_body writes, computed by one wavefront from the ids alone, so that
// the launch needs no plan launch before it. Valid when every expert has one
// item (64 % tm == 0: an expert's at most 64 entries pad to at most 64 rows).
// Item j is then the j-th routed expert in ascending order, its rows start at
// the padded rows of the experts below it, and slot (j) and fields are those
// put_item gives it. per_item: workgroups per item; bid: this workgroup's
// index among the launch's workgroups that take items (a multiple of 8 of
// them, as xcd_logical_block assumes). On return (all lanes):
// *nitems, and for lb >= 0 the item; tok[r] (LDS, kItemRows ints) = the token
// of the item's row r, -1 for pad rows. lb = -1: a surplus workgroup.
__device__ __forceinline__ void wave_plan_item(const int32_t *__restrict__ ids, int nent, int E,
                                               int K, int tm, int nbits, int max_rows,
                                               int per_item, int bid, int *nitems, int *lb,
                                               WorkItem *it, int *tok)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int e = lane < nent ? ids[lane] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t same = __ballot(valid);
    for (int p = 0; p < nbits; ++p) {
        const bool bit = (e >> p) & 1;
        const uint64_t bl = __ballot(bit);
        same &= bit ? bl : ~bl;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(same & below);
    const bool first = valid && rank == 0;
    const int rows = first ? (__popcll(same) + tm - 1) / tm * tm : 0;
    // order among the routed experts and the padded rows below (first lanes)
    const int key = first ? e : 0x7fffffff;
    int ord = 0, rbelow = 0;
    for (int j = 0; j < kWave; ++j) {
        const int kj = __builtin_amdgcn_readlane(key, j);
        const int rj = __builtin_amdgcn_readlane(rows, j);
        if (kj < key) {
            ++ord;
            rbelow += rj;
        }
    }
    const int n = __popcll(__ballot(first));
    const int b = xcd_logical_block(n * per_item, bid);
    *nitems = n;
    *lb = b;
    tok[lane] = -1;  // (kItemRows == kWave) pad rows; the item's entries below
    if (b >= 0) {
        // the first lane of the item's expert (there is one: b / per_item < n)
        const int l = __builtin_amdgcn_readfirstlane(
            (int)__builtin_ctzll(__ballot(first && ord == b / per_item)));
        const int ex = __builtin_amdgcn_readlane(e, l);
        const int row0 = __builtin_amdgcn_readlane(rbelow, l);
        const int r = __builtin_amdgcn_readlane(rows, l);
        it->expert = ex;
        it->row0 = row0;
        it->nrows = min(min(kItemRows, r), max_rows - row0);
        it->run = 1;
        // (after this wavefront's stores of -1 above: its LDS accesses are in order)
        if (valid && e == ex) tok[rank] = lane / K;
    }
}

}  // namespace moe
