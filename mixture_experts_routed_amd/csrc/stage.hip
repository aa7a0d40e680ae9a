// Expert weights in host memory: staging the routed experts into a device
// cache before the grouped FFN.
//
// Source: "#372 Prompt path: an MMQ group's experts gathered in one launch,
// after one wait, released by one event", description (the experts a prompt
// chunk routes to are streamed from host memory into ring slots, and a group
// of them is copied into its slots by one launch), and "Add --moe-mode
// sweep-prefill: streamed expert supply for CPU mul_mat_id", Mechanism (the
// used experts are walked in ascending expert order over their contiguous
// weight slices). There the host issues the copies, so it must learn the
// routed experts first. Here the GPU pulls the weights itself from pinned,
// device-mapped host memory, so the call needs no host synchronisation: after
// the plan, one launch
//  * ranks the routed experts (cnt[e] > 0) in ascending order: expert e gets
//    slot s (every workgroup computes the ranks itself from the E counts, so
//    no workgroup waits for another);
//  * renumbers the work list from experts to slots (workgroup 0), and writes
//    the slot table (slot_of[e], -1 for an expert the call does not route to);
//  * copies the three matrices of each routed expert from host memory into
//    its slots, 16 bytes per lane, 8 loads in flight per lane, grid-strided.
// The grouped FFN then runs unchanged on the cache: a slot has the layout's
// per-expert stride, so the work items' slot numbers address it as expert
// numbers address the full weight arrays.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kStageBlock = 256;
constexpr int kStageUnroll = 8;

__global__ __launch_bounds__(kStageBlock) void k_stage_experts(
    const int32_t *__restrict__ cnt, int E, const int32_t *__restrict__ ctl,
    WorkItem *__restrict__ items, const uint4 *__restrict__ hg, const uint4 *__restrict__ hu,
    const uint4 *__restrict__ hd, int64_t ngu, int64_t ndn, int32_t *__restrict__ slot_of,
    uint4 *__restrict__ cg, uint4 *__restrict__ cu, uint4 *__restrict__ cd)
{
    __shared__ int s_exp[kMaxExperts];   // expert of slot s
    __shared__ int s_slot[kMaxExperts];  // slot of expert e, -1: not routed to
    __shared__ int s_wsum[kStageBlock / kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;

    // ranks of the routed experts, 256 experts at a time
    int nact = 0;
    for (int e0 = 0; e0 < E; e0 += kStageBlock) {
        const int e = e0 + tid;
        const int a = e < E && cnt[e] > 0 ? 1 : 0;
        const int incl = wave_inclusive_scan(a, lane);
        if (lane == kWave - 1) s_wsum[wv] = incl;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int q = 0; q < kStageBlock / kWave; ++q) {
            before += q < wv ? s_wsum[q] : 0;
            total += s_wsum[q];
        }
        if (e < E) {
            const int s = a ? nact + before + incl - 1 : -1;
            s_slot[e] = s;
            if (a) s_exp[s] = e;
        }
        nact += total;
        __syncthreads();  // s_wsum is written again; s_slot / s_exp complete after the loop
    }

    if (blockIdx.x == 0) {
        for (int e = tid; e < E; e += kStageBlock) slot_of[e] = s_slot[e];
        const int nitems = ctl[0];
        for (int i = tid; i < nitems; i += kStageBlock) {
            const int ex = items[i].expert;
            const int s = (unsigned)ex < (unsigned)E ? s_slot[ex] : -1;
            // (an item's expert always has entries; were it not so, the item
            // would compute no rows against slot 0 rather than read outside)
            items[i].expert = s < 0 ? 0 : s;
            if (s < 0) items[i].nrows = 0;
        }
    }

    // the copy: unit u of the nact x (2 ngu + ndn) 16-byte units
    const int64_t per = 2 * ngu + ndn;
    const int64_t nunits = (int64_t)nact * per;
    const int64_t stride = (int64_t)gridDim.x * kStageBlock;
    for (int64_t u0 = (int64_t)blockIdx.x * kStageBlock + tid; u0 < nunits;
         u0 += stride * kStageUnroll) {
        uint4 v[kStageUnroll];
        uint4 *dst[kStageUnroll];
#pragma unroll
        for (int k = 0; k < kStageUnroll; ++k) {
            const int64_t u = u0 + k * stride;
            dst[k] = nullptr;
            if (u >= nunits) continue;
            const int64_t s = u / per;
            int64_t r = u - s * per;
            const int64_t ex = s_exp[s];
            if (r < ngu) {
                v[k] = hg[ex * ngu + r];
                dst[k] = cg + s * ngu + r;
            } else if ((r -= ngu) < ngu) {
                v[k] = hu[ex * ngu + r];
                dst[k] = cu + s * ngu + r;
            } else {
                r -= ngu;
                v[k] = hd[ex * ndn + r];
                dst[k] = cd + s * ndn + r;
            }
        }
#pragma unroll
        for (int k = 0; k < kStageUnroll; ++k)
            if (dst[k]) *dst[k] = v[k];
    }
}

hipError_t launch_stage_experts(const int32_t *cnt, int E, const void *ffn_scratch,
                                const void *hg, const void *hu, const void *hd, size_t bytes_gu,
                                size_t bytes_dn, int64_t max_slots, int32_t *slot_of, void *cg,
                                void *cu, void *cd, hipStream_t s)
{
    const int32_t *ctl = static_cast<const int32_t *>(ffn_scratch);
    WorkItem *items = reinterpret_cast<WorkItem *>(
        static_cast<char *>(const_cast<void *>(ffn_scratch)) + kCtlBytes);
    const int64_t ngu = (int64_t)(bytes_gu / 16), ndn = (int64_t)(bytes_dn / 16);
    // enough workgroups for the most units a call can copy, at most 1024
    const int64_t most = max_slots * (2 * ngu + ndn);
    int64_t nb = (most + (int64_t)kStageBlock * kStageUnroll - 1) / ((int64_t)kStageBlock * kStageUnroll);
    nb = nb < 1 ? 1 : (nb > 1024 ? 1024 : nb);
    hipLaunchKernelGGL(k_stage_experts, dim3((unsigned)nb), dim3(kStageBlock), 0, s, cnt, E, ctl,
                       items, static_cast<const uint4 *>(hg), static_cast<const uint4 *>(hu),
                       static_cast<const uint4 *>(hd), ngu, ndn, slot_of,
                       static_cast<uint4 *>(cg), static_cast<uint4 *>(cu),
                       static_cast<uint4 *>(cd));
    return hipGetLastError();
}

}  // namespace moe
