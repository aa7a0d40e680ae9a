// Host launchers of the routed MoE kernels (internal C++ interface between the
// kernel sources and the C ABI in abi.cpp). Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- plan: histogram, scan + pad fill, placement ----
hipError_t launch_hist(const int32_t *ids, int nent, int E, int nblk, int32_t *bcnt, hipStream_t s);
hipError_t launch_scan(const int32_t *bcnt, int nblk, int E, int K, int tm, int nent, int32_t *cnt,
                       int32_t *eoff, int32_t *boff, int32_t *tiles, int32_t *stok, float *sw,
                       int32_t *meta, hipStream_t s);
hipError_t launch_place(const int32_t *ids, const float *w, int nent, int E, int K, int nblk,
                        const int32_t *eoff, const int32_t *boff, int32_t *stok, float *sw,
                        int32_t *pos, hipStream_t s);
// Whole plan in one launch (each workgroup counts all entries); valid when
// nblk <= plan_fused_max_blocks(). With ffn_scratch != nullptr it also writes
// the grouped FFN's work list (max_items items) for rows capped at max_rows.
int plan_fused_max_blocks();
hipError_t launch_plan_fused(const int32_t *ids, const float *w, int nent, int E, int K, int tm,
                             int nblk, int32_t *cnt, int32_t *eoff, int32_t *boff, int32_t *tiles,
                             int32_t *stok, float *sw, int32_t *pos, int32_t *meta,
                             void *ffn_scratch, int64_t max_items, int64_t max_rows,
                             bool runs_first, hipStream_t s);

// ---- router ----
hipError_t launch_route_topk(const float *logits, int T, int E, int K, int32_t *ids, float *w,
                             hipStream_t s);

// ---- gather and combine ----
hipError_t launch_gather(const void *x, int elem_bytes, int T, int d, const int32_t *stok,
                         const int32_t *meta, int64_t max_rows, void *xs, hipStream_t s);
hipError_t launch_combine(const float *y, int64_t max_rows, const int32_t *pos, int T, int K,
                          int d, float *out, hipStream_t s);
// the combine over compact expert outputs (binary16 rows y16, block exponents yexp)
hipError_t launch_combine_y16(const uint16_t *y16, const int8_t *yexp, int64_t max_rows,
                              const int32_t *pos, int T, int K, int d, float *out, hipStream_t s);

// ---- grouped expert FFN ----
// rows per work item of the grouped GEMMs
int ffn_rows_per_item();
// bound on the number of work items for a plan of max_rows rows
int64_t ffn_max_items(int E, int tm, int64_t max_rows);

// Launch shape of the two grouped GEMMs for a plan bound (host side): K
// splits, grid sizes and the layout of the FFN scratch (item count, work
// items, then the split-K partial planes when a GEMM is split).
struct FfnShape {
    int64_t max_items, max_rows;
    int split_gu, steps_gu;  // gate/up: K splits and K-steps per split
    int split_dn, steps_dn;  // down
    int64_t blocks_gu, blocks_dn;  // workgroups per launch
    // runs of 4 items of the packed 16-bit projections on the 8-wavefront
    // kernel (when not split): whether, and its grids (bound on runs x column
    // blocks)
    bool big_gu, big_dn;
    int64_t blocks_big_gu, blocks_big_dn;
    int64_t plane_gu, plane_dn;    // floats per partial plane
    size_t part_offset;            // byte offset of the partial planes
    size_t scratch_bytes;
};
FfnShape ffn_shape(int E, int tm, int64_t max_rows, int d, int f, int dtype);

// A call of at most one wavefront of entries whose experts each get one work
// item (wave_plan_fits) can be planned inside the gathered gate/up launch:
// every workgroup finds its own work item from the ids, and the launch's first
// workgroup writes the plan's outputs and the work list for the kernels after
// it, as the one-wavefront plan launch would (bit for bit). ids == nullptr:
// the launch reads the work list the plan wrote.
struct WavePlan {
    const int32_t *ids;
    const float *w;
    int nent, E, K, tm, nbits, max_items, max_rows;
    int32_t *cnt, *eoff, *boff, *tiles, *stok;
    float *sw;
    int32_t *pos, *meta;
};
bool wave_plan_fits(int64_t nent, int tm);

// runs_first: the items in runs of 4 first (item_slot), for the big cells
hipError_t launch_worklist(const int32_t *eoff, int E, int64_t max_rows, void *scratch,
                           int64_t max_items, bool runs_first, hipStream_t s);
hipError_t launch_gateup(const FfnShape &z, int dtype, bool packed, const void *xs,
                         const int32_t *stok, const void *wg, const void *wu, int d, int f,
                         const int32_t *meta, const void *scratch, void *h, hipStream_t s);
// gate/up reading row r straight from x[stok[r]] (the gather fused into the
// A-tile loads); x must be smaller than 2 GiB.
// wp != nullptr with wp->ids set: the call is planned inside this launch (WavePlan).
hipError_t launch_gateup_gathered(const FfnShape &z, int dtype, bool packed, const void *x, int T,
                                  const int32_t *stok, const void *wg, const void *wu, int d, int f,
                                  const int32_t *meta, const void *scratch, void *h, hipStream_t s,
                                  const WavePlan *wp = nullptr);
// yexp == nullptr: y is fp32 [rows][d]; otherwise (16-bit types only) y holds
// binary16 rows and yexp [rows][ceil(d / 128)] their block exponents (the
// compact format of common.hpp)
hipError_t launch_down(const FfnShape &z, int dtype, bool packed, const void *h, const void *wd,
                       int d, int f, const int32_t *stok, const float *sw, const int32_t *meta,
                       const void *scratch, void *y, int8_t *yexp, hipStream_t s);

// ---- packed expert weights ----
// bytes of one packed matrix set: gate/up matrices [E][d][f] (gateup = true,
// Kd = d, N = f) or the down matrices [E][f][d] (Kd = f, N = d)
size_t packed_weight_bytes(int E, int Kd, int N, bool gateup, int dtype);
hipError_t launch_pack(int dtype, const void *src, int E, int Kd, int N, bool gateup, void *dst,
                       hipStream_t s);

// Expert weights in host memory (stage.hip): a device cache of S expert slots
// per matrix (bytes_gu per slot for gate and up, bytes_dn for down) and its
// state (hdr[2]: ring hand, experts copied by the last call; slot_of[E];
// exp_of[S]; copy[S]).
struct CacheState {
    int32_t *hdr, *slot_of, *exp_of, *copy;
    void *gate, *up, *down;
    size_t bytes_gu, bytes_dn;
    int E, S;
};
// an empty cache
hipError_t launch_cache_clear(const CacheState &c, hipStream_t s);
// give the routed experts slots (ring order from the hand; resident ones
// kept), renumber the work list in ffn_scratch to slots, and copy the new
// experts' matrices from the device-mapped host pointers hg, hu, hd; max_new
// bounds the experts one call routes to (min(E, T K))
hipError_t launch_cache_stage(const CacheState &c, const int32_t *cnt, const void *ffn_scratch,
                              const void *hg, const void *hu, const void *hd, int64_t max_new,
                              hipStream_t s);

}  // namespace moe
