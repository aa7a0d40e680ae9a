// Router top-k for gfx950: softmax over E logits, the K largest kept and
// renormalised, ids in descending order (equal logits: lower expert id first).
//
// Source: "Round 4 Track C: Prefill MoE Plan ... & Epilogue / Gather Audit",
// section 1 finding 5 and section 3 name route_topk as the kernel that writes
// the routed ids before the plan. The softmax-then-top-k-renormalised rule
// comes from the workload description: the full softmax denominator cancels,
// so weight k = exp(l_k - m) / sum over the K picks of exp(l_j - m), with m the
// largest logit.
//
// One wavefront per token: lane l holds logits l, l+64, ... (E <= 1024), and
// each of the K rounds is one 64-bit wave max over keys that order (value,
// -index) -- an order-preserving image of the float in the high word, the
// inverted index in the low word -- so the winner is the largest logit and, on
// equal logits, the lowest id. NaN logits never compete. The exponentials are
// summed in pick order; lane k keeps pick k (K <= 64) and writes it. The wave
// max runs on DPP lane moves (no LDS round trips), so the winner is uniform
// and its logit is read from the owning lane with readlane.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

// logits per lane: NJ = 2, 4, 8 or 16 (E <= 64 * NJ), a template parameter so
// that the per-round scan of a lane's candidates covers only real experts

// order-preserving map of a non-NaN float to uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t ordered(float v)
{
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// one DPP step of a wave max over 64-bit keys held as (hi, lo) words; lanes
// without a source take key 0, which is below every candidate
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ void key_max_step(uint32_t &hi, uint32_t &lo)
{
    const uint32_t h2 = (uint32_t)dpp_move<CTRL, ROWS>((int)hi, 0);
    const uint32_t l2 = (uint32_t)dpp_move<CTRL, ROWS>((int)lo, 0);
    const bool gt = h2 > hi || (h2 == hi && l2 > lo);
    hi = gt ? h2 : hi;
    lo = gt ? l2 : lo;
}

// largest key of the wave, in every lane (as wave_max: DPP row shifts and
// broadcasts, the total lands in lane 63)
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
    key_max_step<kRowShr + 1>(hi, lo);
    key_max_step<kRowShr + 2>(hi, lo);
    key_max_step<kRowShr + 4>(hi, lo);
    key_max_step<kRowShr + 8>(hi, lo);
    key_max_step<kRowBcast15, 0xa>(hi, lo);
    key_max_step<kRowBcast31, 0xc>(hi, lo);
    hi = __builtin_amdgcn_readlane(hi, kWave - 1);
    lo = __builtin_amdgcn_readlane(lo, kWave - 1);
    return ((uint64_t)hi << 32) | lo;
}

template <int NJ>
__global__ __launch_bounds__(256) void k_route_topk(const float *__restrict__ logits, int T, int E,
                                                    int K, int32_t *__restrict__ ids,
                                                    float *__restrict__ w)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const float *row = logits + (size_t)t * E;
    float v[NJ];
    uint32_t avail = 0;  // bit j: logit lane + 64*j is present, not NaN, not yet picked
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + kWave * j;
        v[j] = e < E ? row[e] : 0.f;
        if (e < E && !__builtin_isnan(v[j])) avail |= 1u << j;
    }
    float m = 0.f, sum = 0.f, my_e = 0.f;
    int my_id = -1;
    for (int k = 0; k < K; ++k) {
        uint64_t key = 0;  // 0: no candidate (below every real key)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if ((avail >> j) & 1u) {
                const uint64_t c = ((uint64_t)ordered(v[j]) << 32) |
                                   (uint32_t)(0xffffffffu - (uint32_t)(lane + kWave * j));
                key = c > key ? c : key;
            }
        key = wave_max_u64(key);
        int id = -1;
        float e_k = 0.f;
        if (key != 0) {
            id = (int)(0xffffffffu - (uint32_t)key);
            const int owner = id & (kWave - 1), slot = id >> 6;
            float val = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) val = (j == slot) ? v[j] : val;
            val = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, val), owner));
            if (lane == owner) avail &= ~(1u << slot);
            if (k == 0) m = val;
            e_k = expf(val - m);
            sum += e_k;  // pick order
        }
        if (lane == k) {
            my_id = id;
            my_e = e_k;
        }
    }
    if (lane < K) {
        ids[(size_t)t * K + lane] = my_id;
        w[(size_t)t * K + lane] = my_id >= 0 ? my_e / sum : 0.f;
    }
}

hipError_t launch_route_topk(const float *logits, int T, int E, int K, int32_t *ids, float *w,
                             hipStream_t s)
{
    const dim3 grid((T + 3) / 4), block(256);
    if (E <= 2 * kWave)
        hipLaunchKernelGGL(k_route_topk<2>, grid, block, 0, s, logits, T, E, K, ids, w);
    else if (E <= 4 * kWave)
        hipLaunchKernelGGL(k_route_topk<4>, grid, block, 0, s, logits, T, E, K, ids, w);
    else if (E <= 8 * kWave)
        hipLaunchKernelGGL(k_route_topk<8>, grid, block, 0, s, logits, T, E, K, ids, w);
    else
        hipLaunchKernelGGL(k_route_topk<16>, grid, block, 0, s, logits, T, E, K, ids, w);
    return hipGetLastError();
}

}  // namespace moe
