// Expert weights in host memory: a device cache of expert slots, filled per
// call with the routed experts that it does not hold yet.
//
// Source: "#372 Prompt path: an MMQ group's experts gathered in one launch,
// after one wait, released by one event", description (the experts a prompt
// chunk routes to are streamed from host memory into a ring of device slots; a
// group of them is copied by one launch; ring entries the routing does not
// use are skipped), and "Add --moe-mode sweep-prefill: streamed expert supply
// for CPU mul_mat_id", Mechanism (the used experts are walked in ascending
// expert order over their contiguous weight slices). There the host issues
// the copies and must first learn the routed experts. Here the GPU decides and
// pulls the weights itself from pinned, device-mapped host memory, so a call
// enqueues and never waits for the GPU. After the plan:
//  * k_cache_assign (one workgroup) keeps the slot of every routed expert that
//    has one, and gives each other routed expert, in ascending expert order,
//    the next free slot of the ring from the hand on (a slot is free unless
//    this call routes to the expert it holds; the expert a slot loses is
//    evicted); the hand moves past the last slot given. It writes the copy list
//    and renumbers the work list from experts to slots;
//  * k_cache_fill copies the three matrices of every listed expert from host
//    memory into its slot, 16 bytes per lane, 8 loads in flight per lane.
// The grouped FFN then runs unchanged on the cache: a slot has the layout's
// per-expert stride, so the work items' slot numbers address it as expert
// numbers address the full weight arrays.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kAssignBlock = 1024;
constexpr int kFillBlock = 256;
constexpr int kFillUnroll = 8;

static_assert(kMaxExperts <= kAssignBlock, "one lane per expert and per ring position");

// Lane tid stands for expert tid and for ring position tid (slot (hand + tid)
// mod S). State: hdr[0] = hand, hdr[1] = experts copied by the last call;
// slot_of[E] (-1: none); exp_of[S] (-1: empty); copy[S] = slot | expert << 16.
__global__ __launch_bounds__(kAssignBlock) void k_cache_assign(
    const int32_t *__restrict__ cnt, int E, int S, const int32_t *__restrict__ ctl,
    WorkItem *__restrict__ items, int32_t *__restrict__ hdr, int32_t *__restrict__ slot_of,
    int32_t *__restrict__ exp_of, int32_t *__restrict__ copy)
{
    constexpr int NW = kAssignBlock / kWave;
    __shared__ int s_slot[kMaxExperts];  // slot of expert e after this call
    __shared__ int s_new[kMaxExperts];   // the r-th new expert
    __shared__ int s_wsum[2][NW];
    __shared__ int s_hand;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;

    // the state before the call (every read of exp_of before the first barrier)
    const int hand = hdr[0];
    const bool routed = tid < E && cnt[tid] > 0;
    // (a slot number outside [0, S) -- a cache made for other sizes -- counts as
    // none, so that no work item can address past the cache)
    const int raw_slot = tid < E ? slot_of[tid] : -1;
    const int old_slot = (unsigned)raw_slot < (unsigned)S ? raw_slot : -1;
    const int isnew = routed && old_slot < 0 ? 1 : 0;
    const int sq = tid < S ? (hand + tid) % S : 0;
    const int sq_exp = tid < S ? exp_of[sq] : -1;
    const bool held = (unsigned)sq_exp < (unsigned)E;
    const int isfree = tid < S && !(held && cnt[sq_exp] > 0) ? 1 : 0;
    const int nw = wave_inclusive_scan(isnew, lane);
    const int nf = wave_inclusive_scan(isfree, lane);
    if (lane == kWave - 1) {
        s_wsum[0][wv] = nw;
        s_wsum[1][wv] = nf;
    }
    if (tid < E) s_slot[tid] = old_slot;
    if (tid == 0) s_hand = hand;
    __syncthreads();
    int before = 0, nnew = 0, fbefore = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        before += w < wv ? s_wsum[0][w] : 0;
        nnew += s_wsum[0][w];
        fbefore += w < wv ? s_wsum[1][w] : 0;
    }
    if (isnew) s_new[before + nw - 1] = tid;
    __syncthreads();
    // the r-th free slot of the ring takes the r-th new expert (S >= the routed
    // experts, so there are enough free slots); its old expert is evicted (not
    // routed by this call, so no other lane writes its entry)
    const int rfree = fbefore + nf - 1;
    if (isfree && rfree < nnew) {
        const int ex = s_new[rfree];
        s_slot[ex] = sq;
        if (held) s_slot[sq_exp] = -1;
        exp_of[sq] = ex;
        copy[rfree] = sq | (ex << 16);
        if (rfree == nnew - 1) s_hand = (sq + 1) % S;
    }
    __syncthreads();
    if (tid < E) slot_of[tid] = s_slot[tid];
    if (tid == 0) {
        hdr[0] = s_hand;
        hdr[1] = nnew;
    }
    const int nitems = ctl[0];
    for (int i = tid; i < nitems; i += kAssignBlock) {
        const int ex = items[i].expert;
        const int s = (unsigned)ex < (unsigned)E ? s_slot[ex] : -1;
        // (an item's expert always has entries, so it has a slot; were it not
        // so, the item would compute no rows against slot 0 rather than read
        // outside the cache)
        items[i].expert = s < 0 ? 0 : s;
        if (s < 0) items[i].nrows = 0;
    }
}

// Copy the listed experts' matrices: unit u of the hdr[1] x (2 ngu + ndn)
// 16-byte units, grid-strided.
__global__ __launch_bounds__(kFillBlock) void k_cache_fill(
    const int32_t *__restrict__ hdr, const int32_t *__restrict__ copy,
    const uint4 *__restrict__ hg, const uint4 *__restrict__ hu, const uint4 *__restrict__ hd,
    int64_t ngu, int64_t ndn, uint4 *__restrict__ cg, uint4 *__restrict__ cu,
    uint4 *__restrict__ cd)
{
    const int ncopy = hdr[1];
    const int64_t per = 2 * ngu + ndn;
    const int64_t nunits = (int64_t)ncopy * per;
    const int64_t stride = (int64_t)gridDim.x * kFillBlock;
    for (int64_t u0 = (int64_t)blockIdx.x * kFillBlock + threadIdx.x; u0 < nunits;
         u0 += stride * kFillUnroll) {
        uint4 v[kFillUnroll];
        uint4 *dst[kFillUnroll];
#pragma unroll
        for (int k = 0; k < kFillUnroll; ++k) {
            const int64_t u = u0 + k * stride;
            dst[k] = nullptr;
            if (u >= nunits) continue;
            const int64_t j = u / per;
            int64_t r = u - j * per;
            const int32_t c = copy[j];
            const int64_t s = c & 0xffff, ex = (uint32_t)c >> 16;
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
        for (int k = 0; k < kFillUnroll; ++k)
            if (dst[k]) *dst[k] = v[k];
    }
}

// An empty cache: hand 0, nothing copied, no slot held.
__global__ __launch_bounds__(kAssignBlock) void k_cache_clear(int32_t *__restrict__ hdr,
                                                             int32_t *__restrict__ slot_of, int E,
                                                             int32_t *__restrict__ exp_of, int S)
{
    const int tid = threadIdx.x;
    if (tid < 2) hdr[tid] = 0;
    if (tid < E) slot_of[tid] = -1;
    if (tid < S) exp_of[tid] = -1;
}

hipError_t launch_cache_clear(const CacheState &c, hipStream_t s)
{
    hipLaunchKernelGGL(k_cache_clear, dim3(1), dim3(kAssignBlock), 0, s, c.hdr, c.slot_of, c.E,
                       c.exp_of, c.S);
    return hipGetLastError();
}

hipError_t launch_cache_stage(const CacheState &c, const int32_t *cnt, const void *ffn_scratch,
                              const void *hg, const void *hu, const void *hd, int64_t max_new,
                              hipStream_t s)
{
    const int32_t *ctl = static_cast<const int32_t *>(ffn_scratch);
    WorkItem *items = reinterpret_cast<WorkItem *>(
        static_cast<char *>(const_cast<void *>(ffn_scratch)) + kCtlBytes);
    hipLaunchKernelGGL(k_cache_assign, dim3(1), dim3(kAssignBlock), 0, s, cnt, c.E, c.S, ctl,
                       items, c.hdr, c.slot_of, c.exp_of, c.copy);
    const int64_t ngu = (int64_t)(c.bytes_gu / 16), ndn = (int64_t)(c.bytes_dn / 16);
    // enough workgroups for the most units a call can copy, at most 1024
    const int64_t most = max_new * (2 * ngu + ndn);
    const int64_t unit = (int64_t)kFillBlock * kFillUnroll;
    int64_t nb = (most + unit - 1) / unit;
    nb = nb < 1 ? 1 : (nb > 1024 ? 1024 : nb);
    hipLaunchKernelGGL(k_cache_fill, dim3((unsigned)nb), dim3(kFillBlock), 0, s, c.hdr, c.copy,
                       static_cast<const uint4 *>(hg), static_cast<const uint4 *>(hu),
                       static_cast<const uint4 *>(hd), ngu, ndn, static_cast<uint4 *>(c.gate),
                       static_cast<uint4 *>(c.up), static_cast<uint4 *>(c.down));
    return hipGetLastError();
}

}  // namespace moe
