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

constexpr int kMT = kItemRows / 16;     // 16-row m-tiles per work item
constexpr int kWavesPerBlock = 4;

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

// ---- raw buffer loads -----------------------------------------------------
// A buffer resource covering exactly one operand range: loads past its end
// return zeros without touching memory (range-checked by the hardware), which
// zero-fills the K tail of the weights and the rows past a work item's end.
// Word 3 = 0x00020000: raw (untyped) buffer on gfx9-family GPUs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Cache policy of a buffer load: 0 = default; kNT = non-temporal (the weights
// are read exactly once, so they should not displace the reused row tiles).
constexpr int kNT = 2;

template <int BYTES, int POLICY = 0> struct Ld;
template <int POLICY> struct Ld<8, POLICY> {
    typedef uint2 type;
    static __device__ __forceinline__ uint2 run(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s)
    {
        return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, v, s, POLICY));
    }
};
template <int POLICY> struct Ld<16, POLICY> {
    typedef uint4 type;
    static __device__ __forceinline__ uint4 run(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s)
    {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, v, s, POLICY));
    }
};

// stores of outputs that this kernel does not read again: non-temporal
__device__ __forceinline__ void store_nt(float4 *p, float4 v)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(f4{v.x, v.y, v.z, v.w}, reinterpret_cast<f4 *>(p));
}
__device__ __forceinline__ void store_nt(uint2 *p, uint2 v)
{
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u2{v.x, v.y}, reinterpret_cast<u2 *>(p));
}

// ---- per element type: MFMA and conversion -------------------------------
template <typename T> struct Elt;

template <> struct Elt<_Float16> {
    static constexpr int KR = 8;  // K-values per lane per MFMA
    static __device__ __forceinline__ float4_t mfma(uint4 a, uint4 b, float4_t c)
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

template <> struct Elt<__bf16> {
    static constexpr int KR = 8;
    static __device__ __forceinline__ float4_t mfma(uint4 a, uint4 b, float4_t c)
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

template <> struct Elt<float> {
    static constexpr int KR = 4;
};

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 16-bit B operand: 8 consecutive K-rows of NPL columns each (row i = K-value
// i). Column c of them, as one MFMA operand (element i = K-row i).
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

__device__ __forceinline__ uint32_t word(const uint4 &v, int q)
{
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

__device__ __forceinline__ float lanef(const uint4 &v, int q)
{
    return __builtin_bit_cast(float, word(v, q));
}

// Pipeline depth for NMT m-tiles: stage = 32 B-operand + 4 A-operand VGPRs,
// accumulators = 32*NMT VGPRs; S stages + accumulators stay <= ~232.
constexpr int stages_for(int nmt) { return nmt >= 4 ? 2 : nmt == 3 ? 3 : nmt == 2 ? 4 : 5; }

// Shared A tile of one K-step: 64 rows x 32 K (16-bit) or 64 rows x 16 K
// (fp32), 64 bytes per row, double-buffered: 2 x 4 KB of LDS per workgroup.
constexpr int kATileBytes = kItemRows * 64;

// A workgroup of 4 wavefronts computes one work item (<= 64 rows) against 4
// adjacent column slices of 16*NPL columns, one slice per wavefront.
//  * A (the item's rows) is shared: per K-step each wavefront loads 16 rows x
//    64 bytes (one 16-byte load per lane) into registers, writes them to an LDS
//    slot, and after one barrier every wavefront reads its MFMA A-fragments
//    from LDS. One copy of A per workgroup instead of one per wavefront.
//  * B (the weights) is private to each wavefront: lane l supplies MFMA column
//    (l & 15) and K-group (l >> 4); it loads KR K-rows x NPL columns of each
//    weight matrix per step (16 lanes cover one 16*NPL-column row segment) and
//    transposes them in registers, so MFMA c produces the logical columns
//    NPL*j + c, j = 0..15.
//  * S-stage register ring: the loads of step s+S-1 are issued before the
//    MFMAs of step s; the loop body is straight-line code, so they stay in
//    flight. The per-step barrier keeps the 4 wavefronts in step, so together
//    they read 4 adjacent row segments of every weight row.
// GATHERED (gate/up only): A is the token activation x [a_rows][Kd] and row r
// of the item reads x[stok[r]] -- the gather fused into the A-tile loads.
template <typename T, bool GATEUP, bool GATHERED, int NPL, int NMT>
__device__ __forceinline__ void wave_gemm(const T *__restrict__ A, int a_rows,
                                          const T *__restrict__ B0,
                                          const T *__restrict__ B1, int Kd, int N, WorkItem it,
                                          int slice, const int32_t *__restrict__ stok,
                                          const float *__restrict__ sw, void *__restrict__ out,
                                          uint4 *__restrict__ a_lds, float2 *__restrict__ rinfo)
{
    constexpr int ES = sizeof(T);
    constexpr int KR = Elt<T>::KR;
    constexpr int KSTEP = 4 * KR;
    constexpr int NMAT = 2;       // two B streams (see above)
    constexpr int LB = NPL * ES;  // bytes per lane per row
    typedef typename Ld<LB>::type RowT;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int nq = lane & 15, kg = lane >> 4;
    // GATEUP: slice = 16*NPL columns of both W_gate and W_up. Down: slice =
    // 2*16*NPL columns of W_down, as two halves 16*NPL columns apart, so that
    // each fp32 store instruction of the epilogue covers whole 64-byte runs.
    constexpr int SW = GATEUP ? 16 * NPL : 32 * NPL;  // columns per slice
    constexpr int HALF = GATEUP ? 0 : 16 * NPL;       // column offset of stream 1
    const int col = slice * SW + NPL * nq;
    const bool slice_ok = slice * SW < N;  // wave-uniform

    // operand ranges: this expert's weight matrices (empty for a surplus
    // slice: its loads return zeros without memory traffic), this item's rows
    const size_t wofs = (size_t)it.expert * Kd * N;
    const uint32_t wbytes = slice_ok ? (uint32_t)((size_t)Kd * N * ES) : 0u;
    const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(B0 + wofs, wbytes);
    // (Kd*N >= 64 >= HALF, so the second range never underflows; readfirstlane
    // keeps the wave-uniform value in an SGPR)
    const uint32_t wbytes1 = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(slice_ok ? (uint32_t)((size_t)Kd * N * ES - (size_t)HALF * ES) : 0u));
    const __amdgpu_buffer_rsrc_t rb1 =
        GATEUP ? make_rsrc(B1 + wofs, wbytes) : make_rsrc(B0 + wofs + HALF, wbytes1);
    const uint32_t rowb = (uint32_t)N * ES;  // bytes per weight row
    const uint32_t vcol = (uint32_t)col * ES;
    // this thread's share of the A tile: row tid/4, 16-byte chunk tid%4
    const int arow = tid >> 2, achunk = (tid & 3) * (16 / ES);
    __amdgpu_buffer_rsrc_t ra;
    uint32_t va0;
    if constexpr (GATHERED) {
        // all of x (< 2 GiB, checked by the host); a pad row (token -1) or a
        // row past the item starts at 2^31, outside the range: it reads zeros
        ra = make_rsrc(A, (uint32_t)((size_t)a_rows * Kd * ES));
        const int t = arow < it.nrows ? stok[it.row0 + arow] : -1;
        va0 = (unsigned)t < (unsigned)a_rows ? (uint32_t)t * (uint32_t)Kd * ES : 0x80000000u;
    } else {
        ra = make_rsrc(A + (size_t)it.row0 * Kd, (uint32_t)((size_t)it.nrows * Kd * ES));
        va0 = (uint32_t)arow * (uint32_t)Kd * ES;
    }

    if constexpr (!GATEUP) {
        // router weight and token of the item's rows for the epilogue (made
        // visible to all wavefronts by the barriers of the K loop)
        if (tid < kItemRows) {
            const bool ok = tid < it.nrows;
            const int64_t r = it.row0 + (ok ? tid : 0);
            rinfo[tid] = make_float2(ok ? sw[r] : 0.f, __int_as_float(ok ? stok[r] : -1));
        }
    }

    float4_t acc[NMAT][NMT][NPL];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int c = 0; c < NPL; ++c) acc[m][mt][c] = float4_t{0.f, 0.f, 0.f, 0.f};

    struct Stage {
        RowT b[NMAT][KR];
        uint4 a;
    };
    auto load = [&](Stage &st, int k0) {
        const int kk = k0 + KR * kg;
        const uint32_t vb = vcol + (uint32_t)kk * rowb;
#pragma unroll
        for (int i = 0; i < KR; ++i) st.b[0][i] = Ld<LB, kNT>::run(rb0, vb, (uint32_t)i * rowb);
#pragma unroll
        for (int i = 0; i < KR; ++i) st.b[1][i] = Ld<LB, kNT>::run(rb1, vb, (uint32_t)i * rowb);
        // K past the end: the weights read as zero; zero A too so that no
        // non-finite value of a neighbouring row can leak in as 0 * inf.
        const int ka = k0 + achunk;
        const uint32_t am = ka < Kd ? 0xffffffffu : 0u;
        const uint4 v = Ld<16>::run(ra, va0 + (uint32_t)ka * ES, 0u);
        st.a = make_uint4(v.x & am, v.y & am, v.z & am, v.w & am);
    };
    auto compute = [&](const Stage &st, int step) {
        uint4 *slot = a_lds + (step & 1) * (kATileBytes / 16);
        slot[tid] = st.a;
        __syncthreads();
        uint4 af[NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) af[mt] = slot[(16 * mt + nq) * 4 + kg];
        if constexpr (ES == 2) {
#pragma unroll
            for (int c = 0; c < NPL; ++c) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    const uint4 fb = column_of_rows(st.b[m], c);
#pragma unroll
                    for (int mt = 0; mt < NMT; ++mt)
                        acc[m][mt][c] = Elt<T>::mfma(af[mt], fb, acc[m][mt][c]);
                }
            }
        } else {
            // fp32: sub-step q uses K = k0 + 4*kg + q in both operands
#pragma unroll
            for (int q = 0; q < KR; ++q)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int c = 0; c < NPL; ++c) {
                        const float b = lanef(st.b[m][q], c);
#pragma unroll
                        for (int mt = 0; mt < NMT; ++mt)
                            acc[m][mt][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                lanef(af[mt], q), b, acc[m][mt][c], 0, 0, 0);
                    }
        }
    };

    constexpr int S = stages_for(NMT);
    const int nsteps = (Kd + KSTEP - 1) / KSTEP;
    Stage st[S];
#pragma unroll
    for (int j = 0; j < S - 1; ++j) load(st[j], j * KSTEP);
    for (int s = 0; s < nsteps; s += S) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            // steps past the end load zero weights (no memory traffic) and add 0
            load(st[(j + S - 1) % S], (s + j + S - 1) * KSTEP);
            __builtin_amdgcn_sched_barrier(0);
            compute(st[j], s + j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Epilogue: acc[m][mt][c][r] is the output at row 16*mt + 4*kg + r of the
    // item and column col + c.
    if (col >= N) return;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = 16 * mt + 4 * kg + r;
            if (rl >= it.nrows) continue;
            const int64_t row = it.row0 + rl;
            if constexpr (GATEUP) {
                float hv[NPL];
#pragma unroll
                for (int c = 0; c < NPL; ++c) hv[c] = silu(acc[0][mt][c][r]) * acc[1][mt][c][r];
                T *H = static_cast<T *>(out) + row * N + col;
                if constexpr (ES == 2) {
                    static_assert(NPL == 4, "16-bit gate/up stores 4 columns per lane");
                    store_nt(reinterpret_cast<uint2 *>(H),
                             make_uint2(Elt<T>::pack2(hv[0], hv[1]), Elt<T>::pack2(hv[2], hv[3])));
                } else {
                    static_assert(NPL == 4, "fp32 gate/up stores 4 columns per lane");
                    store_nt(reinterpret_cast<float4 *>(H), make_float4(hv[0], hv[1], hv[2], hv[3]));
                }
            } else {
                static_assert(NPL == 4, "down stores 4 + 4 columns per lane");
                const float2 ri = rinfo[rl];
                if (__float_as_int(ri.y) < 0) continue;  // pad rows are never combined
                const float g = ri.x;
                float *Y = static_cast<float *>(out) + row * N + col;
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
                    if (col + m * HALF < N)
                        store_nt(reinterpret_cast<float4 *>(Y + m * HALF),
                                 make_float4(g * acc[m][mt][0][r], g * acc[m][mt][1][r],
                                             g * acc[m][mt][2][r], g * acc[m][mt][3][r]));
            }
        }
    }
}

// One workgroup per (work item, group of 4 column slices of 16*NPL).
// Kd = reduction length (d for gate/up, f for down); N = output columns (f for
// gate/up, d for down). GATEUP: B0 = W_gate, B1 = W_up, out = H (type T).
// Otherwise: B0 = W_down, out = Y (fp32), stok/sw used in the epilogue.
template <typename T, bool GATEUP, bool GATHERED, int NPL>
__global__ __launch_bounds__(256, 2) void k_expert_gemm(
    const T *__restrict__ A, int a_rows, const T *__restrict__ B0, const T *__restrict__ B1,
    int Kd, int N,
    const int32_t *__restrict__ ctl, const WorkItem *__restrict__ items,
    const int32_t *__restrict__ stok, const float *__restrict__ sw, void *__restrict__ out)
{
    __shared__ uint4 a_lds[2 * kATileBytes / 16];
    __shared__ float2 rinfo[kItemRows];
    constexpr int SW = GATEUP ? 16 * NPL : 32 * NPL;      // columns per slice
    const int ngroups = (N + 4 * SW - 1) / (4 * SW);      // slice groups per item
    const int lb = xcd_logical_block(ctl[0] * ngroups);
    if (lb < 0) return;  // whole workgroup: no barrier reached
    const WorkItem it = items[lb / ngroups];
    // wave-uniform by construction, so the buffer descriptors live in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = (lb % ngroups) * kWavesPerBlock + wave;
    switch ((it.nrows + 15) >> 4) {  // m-tiles of this item (uniform per workgroup)
    case 1: wave_gemm<T, GATEUP, GATHERED, NPL, 1>(A, a_rows, B0, B1, Kd, N, it, slice, stok, sw, out, a_lds, rinfo); break;
    case 2: wave_gemm<T, GATEUP, GATHERED, NPL, 2>(A, a_rows, B0, B1, Kd, N, it, slice, stok, sw, out, a_lds, rinfo); break;
    case 3: wave_gemm<T, GATEUP, GATHERED, NPL, 3>(A, a_rows, B0, B1, Kd, N, it, slice, stok, sw, out, a_lds, rinfo); break;
    default: wave_gemm<T, GATEUP, GATHERED, NPL, kMT>(A, a_rows, B0, B1, Kd, N, it, slice, stok, sw, out, a_lds, rinfo); break;
    }
}

// columns per lane and B stream: 4 (gate/up: 64 columns of both matrices per
// wave; down: 2 x 64 columns of W_down per wave)
template <typename T> constexpr int npl_down() { return 4; }
constexpr int kNplGateUp = 4;

static unsigned gemm_blocks(int64_t max_items, int N, int slice_cols)
{
    int64_t blocks = max_items * ((N + 4 * slice_cols - 1) / (4 * slice_cols));
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
static hipError_t gateup_t(const void *a, int a_rows, const int32_t *stok, const void *wg,
                           const void *wu, int d, int f, const void *scratch, int64_t max_items,
                           void *h, hipStream_t s)
{
    const int32_t *ctl = static_cast<const int32_t *>(scratch);
    const WorkItem *items =
        reinterpret_cast<const WorkItem *>(static_cast<const char *>(scratch) + kCtlBytes);
    const dim3 grid(gemm_blocks(max_items, f, 16 * kNplGateUp));
    if (stok)  // rows gathered from x through stok
        hipLaunchKernelGGL((k_expert_gemm<T, true, true, kNplGateUp>), grid, dim3(256), 0, s,
                           static_cast<const T *>(a), a_rows, static_cast<const T *>(wg),
                           static_cast<const T *>(wu), d, f, ctl, items, stok, nullptr, h);
    else
        hipLaunchKernelGGL((k_expert_gemm<T, true, false, kNplGateUp>), grid, dim3(256), 0, s,
                           static_cast<const T *>(a), 0, static_cast<const T *>(wg),
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
    hipLaunchKernelGGL((k_expert_gemm<T, false, false, npl_down<T>()>),
                       dim3(gemm_blocks(max_items, d, 32 * npl_down<T>())), dim3(256), 0, s,
                       static_cast<const T *>(h), 0, static_cast<const T *>(wd), nullptr, f, d, ctl,
                       items, stok, sw, static_cast<void *>(y));
    return hipGetLastError();
}

hipError_t launch_gateup(int dtype, const void *xs, const void *wg, const void *wu, int d, int f,
                         const void *scratch, int64_t max_items, void *h, hipStream_t s)
{
    if (dtype == 1) return gateup_t<_Float16>(xs, 0, nullptr, wg, wu, d, f, scratch, max_items, h, s);
    if (dtype == 2) return gateup_t<__bf16>(xs, 0, nullptr, wg, wu, d, f, scratch, max_items, h, s);
    return gateup_t<float>(xs, 0, nullptr, wg, wu, d, f, scratch, max_items, h, s);
}

hipError_t launch_gateup_gathered(int dtype, const void *x, int T, const int32_t *stok,
                                  const void *wg, const void *wu, int d, int f, const void *scratch,
                                  int64_t max_items, void *h, hipStream_t s)
{
    if (dtype == 1) return gateup_t<_Float16>(x, T, stok, wg, wu, d, f, scratch, max_items, h, s);
    if (dtype == 2) return gateup_t<__bf16>(x, T, stok, wg, wu, d, f, scratch, max_items, h, s);
    return gateup_t<float>(x, T, stok, wg, wu, d, f, scratch, max_items, h, s);
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
