// Grouped expert FFN for gfx950 on the expert-sorted rows of the routing plan:
//   gate/up:  H = D( silu(XS_e W_gate[e]) * (XS_e W_up[e]) )   (SwiGLU in the epilogue)
//   down:     Y = sw * (H_e W_down[e])                          (fp32, weight in the epilogue)
//
// Sources: "Batched resident MoE experts on Apple Silicon: a flat parallel
// expert pass", section 1 -- per (token, expert, weight) job: gate/up
// projection, gated activation, weighted down projection; "Round 4 Track C:
// Prefill MoE Plan ... & Epilogue / Gather Audit", section 1, finding 5 --
// the SwiGLU output is kept in half precision, and section 2 -- grouped
// GEMMs over tm-row tiles dominate the layer's time.
//
// Design (MI355X): at 512 experts x ~48 rows each, the weights (6 GB at the
// prefill shape) are streamed once and every weight element meets only a few
// dozen rows, so these GEMMs are bound by HBM, not by the matrix cores.
//  * Work unit = one wavefront: (work item, 64-column slice of the output).
//    A work item is one expert's run of up to 64 rows, so each expert's
//    weights are read from HBM once (experts with more rows get more items).
//  * Matrix cores: v_mfma_f32_16x16x32_{f16,bf16} (v_mfma_f32_16x16x4_f32 for
//    fp32). The weights are row-major [K][N] (N contiguous) but an MFMA lane
//    needs 8 consecutive K of one column. Each lane loads 8 K-rows x 4
//    columns (8-byte loads; 16 lanes cover one 128-byte row segment) and
//    transposes the 8x4 block in registers into 4 B-fragments: fragment c
//    feeds MFMA c, whose 16 columns are the logical columns 4*j + c of the
//    slice. No LDS staging, no repacking of the weights by the caller.
//  * A operand rows (16-byte loads of 8 K) come straight from global memory;
//    the 12-40 waves that share an expert's rows sit on one XCD (see
//    xcd_logical_block), so they hit that XCD's L2.
//  * Loads of K-step s+1 are issued before the MFMAs of step s.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kMT = 4;                  // 16-row m-tiles per work item
constexpr int kItemRows = 16 * kMT;     // rows per work item
constexpr int kNPW = 64;                // output columns per wavefront
constexpr int kWavesPerBlock = 4;
constexpr size_t kCtlBytes = 256;       // scratch header (item count)

int ffn_rows_per_item() { return kItemRows; }

int64_t ffn_max_items(int E, int tm, int64_t max_rows)
{
    const int64_t per_tile = (max_rows + tm - 1) / tm;
    return max_rows / kItemRows + 1 + (E < per_tile ? E : per_tile);
}

size_t ffn_scratch_bytes(int E, int tm, int64_t max_rows)
{
    return kCtlBytes + (size_t)ffn_max_items(E, tm, max_rows) * sizeof(WorkItem);
}

// Work list: each expert's row range [eoff[e], eoff[e+1]) cut into items of at
// most kItemRows rows, in ascending expert order. Ranges are clamped to
// [0, max_rows] so that made-up offsets cannot lead outside the buffers.
__global__ __launch_bounds__(1024) void k_worklist(const int32_t *__restrict__ eoff, int E,
                                                   int64_t max_rows, int32_t *__restrict__ ctl,
                                                   WorkItem *__restrict__ items, int max_items)
{
    __shared__ int s_sum[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int r0 = 0, rows = 0;
    if (tid < E) {
        int64_t a = eoff[tid], b = eoff[tid + 1];
        a = a < 0 ? 0 : (a > max_rows ? max_rows : a);
        b = b < a ? a : (b > max_rows ? max_rows : b);
        r0 = (int)a;
        rows = (int)(b - a);
    }
    const int n = (rows + kItemRows - 1) / kItemRows;
    const int incl = wave_inclusive_scan(n, lane);
    if (lane == 63) s_sum[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int v = s_sum[q];
        before += (q < wv) ? v : 0;
        total += v;
    }
    const int start = before + incl - n;
    for (int q = 0; q < n; ++q) {
        const int idx = start + q;
        if (idx < max_items) {
            WorkItem it;
            it.expert = tid;
            it.row0 = r0 + q * kItemRows;
            it.nrows = min(kItemRows, rows - q * kItemRows);
            it.pad = 0;
            items[idx] = it;
        }
    }
    if (tid == 0) ctl[0] = min(total, max_items);
}

template <typename T> struct Mfma;

template <> struct Mfma<_Float16> {
    static __device__ __forceinline__ float4_t run(uint4 a, uint4 b, float4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi)
    {
        const _Float16 l = (_Float16)lo, h = (_Float16)hi;
        return (uint32_t)__builtin_bit_cast(uint16_t, l) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
    }
};

template <> struct Mfma<__bf16> {
    static __device__ __forceinline__ float4_t run(uint4 a, uint4 b, float4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi)
    {
        const __bf16 l = (__bf16)lo, h = (__bf16)hi;  // round to nearest even
        return (uint32_t)__builtin_bit_cast(uint16_t, l) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
    }
};

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Column c (0..3) of 8 consecutive K-rows, each row holding 4 consecutive
// 16-bit columns (.x = cols 0,1; .y = cols 2,3): 8 K-values of one column as
// an MFMA operand (element j = K-row j).
__device__ __forceinline__ uint4 column_of_rows(const uint2 (&r)[8], int c)
{
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t lo = (c < 2) ? r[2 * p].x : r[2 * p].y;
        const uint32_t hi = (c < 2) ? r[2 * p + 1].x : r[2 * p + 1].y;
        o[p] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// One wavefront per (work item, 64-column slice). Kd = reduction length
// (d for gate/up, f for down); N = output columns (f for gate/up, d for down).
// GATEUP: B0 = W_gate, B1 = W_up, out = H (type T). Otherwise: B0 = W_down,
// out = Y (fp32), stok/sw used in the epilogue.
template <typename T, bool GATEUP>
__global__ __launch_bounds__(256, 2) void k_expert_gemm(
    const T *__restrict__ A, const T *__restrict__ B0, const T *__restrict__ B1, int Kd, int N,
    const int32_t *__restrict__ ctl, const WorkItem *__restrict__ items,
    const int32_t *__restrict__ stok, const float *__restrict__ sw, void *__restrict__ out)
{
    const int nslices = (N + kNPW - 1) / kNPW;
    const int nunits = ctl[0] * nslices;
    const int lb = xcd_logical_block((nunits + kWavesPerBlock - 1) / kWavesPerBlock);
    if (lb < 0) return;
    const int unit = lb * kWavesPerBlock + (threadIdx.x >> 6);
    if (unit >= nunits) return;

    const int lane = threadIdx.x & 63;
    const int nq = lane & 15;  // MFMA row (A) / column (B) index of this lane
    const int kg = lane >> 4;  // which group of K-values this lane supplies
    const WorkItem it = items[unit / nslices];
    const int slice = unit % nslices;
    const int nrows = it.nrows;
    const int nmt = (nrows + 15) >> 4;
    const int col = slice * kNPW + 4 * nq;
    const bool colv = col < N;

    const T *arow[kMT];
    bool av[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        const int rl = 16 * mt + nq;
        av[mt] = rl < nrows;
        arow[mt] = A + (int64_t)(it.row0 + (av[mt] ? rl : 0)) * Kd;
    }
    const int64_t wbase = (int64_t)it.expert * Kd * N + (colv ? col : 0);
    const T *b0 = B0 + wbase;
    const T *b1 = GATEUP ? B1 + wbase : B0;

    float4_t acc0[kMT][4], acc1[kMT][4];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            acc0[mt][c] = float4_t{0.f, 0.f, 0.f, 0.f};
            acc1[mt][c] = float4_t{0.f, 0.f, 0.f, 0.f};
        }

    if constexpr (sizeof(T) == 2) {
        constexpr int KSTEP = 32;
        struct Stage {
            uint2 g[8], u[8];
            uint4 a[kMT];
        };
        auto load = [&](Stage &st, int k0) {
            const int kk = k0 + 8 * kg;
            const bool kv = kk < Kd;
            const int kc = kv ? kk : 0;
            const bool bv = kv && colv;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint2 v = *reinterpret_cast<const uint2 *>(b0 + (int64_t)(kc + i) * N);
                st.g[i] = bv ? v : make_uint2(0u, 0u);
            }
            if constexpr (GATEUP) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(b1 + (int64_t)(kc + i) * N);
                    st.u[i] = bv ? v : make_uint2(0u, 0u);
                }
            }
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
                if (mt < nmt) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(arow[mt] + kc);
                    st.a[mt] = (kv && av[mt]) ? v : make_uint4(0u, 0u, 0u, 0u);
                }
        };
        auto compute = [&](const Stage &st) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 fg = column_of_rows(st.g, c);
                uint4 fu = fg;
                if constexpr (GATEUP) fu = column_of_rows(st.u, c);
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
                    if (mt < nmt) {
                        acc0[mt][c] = Mfma<T>::run(st.a[mt], fg, acc0[mt][c]);
                        if constexpr (GATEUP) acc1[mt][c] = Mfma<T>::run(st.a[mt], fu, acc1[mt][c]);
                    }
            }
        };
        const int nsteps = (Kd + KSTEP - 1) / KSTEP;
        Stage s0, s1;
        load(s0, 0);
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
            load(s1, (s + 1) * KSTEP);
            compute(s0);
            if (s + 2 < nsteps) load(s0, (s + 2) * KSTEP);
            compute(s1);
        }
        if (s < nsteps) compute(s0);
    } else {
        // fp32: v_mfma_f32_16x16x4_f32, one K-value per lane per MFMA. A lane
        // loads 4 consecutive K of its A row and the 4 matching B rows; sub-step
        // q uses K = k0 + 4*kg + q in both operands.
        constexpr int KSTEP = 16;
        struct Stage {
            float4 g[4], u[4];
            float4 a[kMT];
        };
        auto load = [&](Stage &st, int k0) {
            const int kk = k0 + 4 * kg;
            const bool kv = kk < Kd;
            const int kc = kv ? kk : 0;
            const bool bv = kv && colv;
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = *reinterpret_cast<const float4 *>(b0 + (int64_t)(kc + q) * N);
                st.g[q] = bv ? v : z;
                if constexpr (GATEUP) {
                    const float4 w = *reinterpret_cast<const float4 *>(b1 + (int64_t)(kc + q) * N);
                    st.u[q] = bv ? w : z;
                }
            }
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
                if (mt < nmt) {
                    const float4 v = *reinterpret_cast<const float4 *>(arow[mt] + kc);
                    st.a[mt] = (kv && av[mt]) ? v : z;
                }
        };
        auto compute = [&](const Stage &st) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float gq[4] = {st.g[q].x, st.g[q].y, st.g[q].z, st.g[q].w};
                const float uq[4] = {st.u[q].x, st.u[q].y, st.u[q].z, st.u[q].w};
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
                    if (mt < nmt) {
                        const float aq = (q == 0) ? st.a[mt].x
                                       : (q == 1) ? st.a[mt].y
                                       : (q == 2) ? st.a[mt].z
                                                  : st.a[mt].w;
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            acc0[mt][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, gq[c], acc0[mt][c], 0, 0, 0);
                            if constexpr (GATEUP)
                                acc1[mt][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, uq[c], acc1[mt][c], 0, 0, 0);
                        }
                    }
            }
        };
        const int nsteps = (Kd + KSTEP - 1) / KSTEP;
        Stage s0, s1;
        load(s0, 0);
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
            load(s1, (s + 1) * KSTEP);
            compute(s0);
            if (s + 2 < nsteps) load(s0, (s + 2) * KSTEP);
            compute(s1);
        }
        if (s < nsteps) compute(s0);
    }

    // Epilogue. acc[mt][c][r] is the output at row 16*mt + 4*kg + r of the
    // item and column col + c.
    if (!colv) return;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
        if (mt >= nmt) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = 16 * mt + 4 * kg + r;
            if (rl >= nrows) continue;
            const int64_t row = it.row0 + rl;
            if constexpr (GATEUP) {
                float hv[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) hv[c] = silu(acc0[mt][c][r]) * acc1[mt][c][r];
                T *H = static_cast<T *>(out) + row * N + col;
                if constexpr (sizeof(T) == 2) {
                    *reinterpret_cast<uint2 *>(H) =
                        make_uint2(Mfma<T>::pack2(hv[0], hv[1]), Mfma<T>::pack2(hv[2], hv[3]));
                } else {
                    *reinterpret_cast<float4 *>(H) = make_float4(hv[0], hv[1], hv[2], hv[3]);
                }
            } else {
                if (stok[row] < 0) continue;  // pad rows are never combined
                const float s = sw[row];
                float *Y = static_cast<float *>(out) + row * N + col;
                *reinterpret_cast<float4 *>(Y) =
                    make_float4(s * acc0[mt][0][r], s * acc0[mt][1][r], s * acc0[mt][2][r],
                                s * acc0[mt][3][r]);
            }
        }
    }
}

static unsigned gemm_blocks(int64_t max_items, int N)
{
    const int64_t units = max_items * ((N + kNPW - 1) / kNPW);
    int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
    blocks = (blocks + 7) / 8 * 8;  // whole rounds over the 8 XCDs
    return (unsigned)blocks;
}

hipError_t launch_worklist(const int32_t *eoff, int E, int64_t max_rows, void *scratch,
                           int64_t max_items, hipStream_t s)
{
    int32_t *ctl = static_cast<int32_t *>(scratch);
    WorkItem *items = reinterpret_cast<WorkItem *>(static_cast<char *>(scratch) + kCtlBytes);
    hipLaunchKernelGGL(k_worklist, dim3(1), dim3(1024), 0, s, eoff, E, max_rows, ctl, items,
                       (int)max_items);
    return hipGetLastError();
}

template <typename T>
static hipError_t gateup_t(const void *xs, const void *wg, const void *wu, int d, int f,
                           const void *scratch, int64_t max_items, void *h, hipStream_t s)
{
    const int32_t *ctl = static_cast<const int32_t *>(scratch);
    const WorkItem *items =
        reinterpret_cast<const WorkItem *>(static_cast<const char *>(scratch) + kCtlBytes);
    hipLaunchKernelGGL((k_expert_gemm<T, true>), dim3(gemm_blocks(max_items, f)), dim3(256), 0, s,
                       static_cast<const T *>(xs), static_cast<const T *>(wg),
                       static_cast<const T *>(wu), d, f, ctl, items, nullptr, nullptr, h);
    return hipGetLastError();
}

template <typename T>
static hipError_t down_t(const void *h, const void *wd, int d, int f, const int32_t *stok,
                         const float *sw, const void *scratch, int64_t max_items, float *y,
                         hipStream_t s)
{
    const int32_t *ctl = static_cast<const int32_t *>(scratch);
    const WorkItem *items =
        reinterpret_cast<const WorkItem *>(static_cast<const char *>(scratch) + kCtlBytes);
    hipLaunchKernelGGL((k_expert_gemm<T, false>), dim3(gemm_blocks(max_items, d)), dim3(256), 0, s,
                       static_cast<const T *>(h), static_cast<const T *>(wd), nullptr, f, d, ctl,
                       items, stok, sw, static_cast<void *>(y));
    return hipGetLastError();
}

hipError_t launch_gateup(int dtype, const void *xs, const void *wg, const void *wu, int d, int f,
                         const void *scratch, int64_t max_items, void *h, hipStream_t s)
{
    if (dtype == 1) return gateup_t<_Float16>(xs, wg, wu, d, f, scratch, max_items, h, s);
    if (dtype == 2) return gateup_t<__bf16>(xs, wg, wu, d, f, scratch, max_items, h, s);
    return gateup_t<float>(xs, wg, wu, d, f, scratch, max_items, h, s);
}

hipError_t launch_down(int dtype, const void *h, const void *wd, int d, int f, const int32_t *stok,
                       const float *sw, const void *scratch, int64_t max_items, float *y,
                       hipStream_t s)
{
    if (dtype == 1) return down_t<_Float16>(h, wd, d, f, stok, sw, scratch, max_items, y, s);
    if (dtype == 2) return down_t<__bf16>(h, wd, d, f, stok, sw, scratch, max_items, y, s);
    return down_t<float>(h, wd, d, f, stok, sw, scratch, max_items, y, s);
}

}  // namespace moe
