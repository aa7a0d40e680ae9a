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
//  * Work list: each expert's rows cut into items of <= 64 rows. A workgroup
//    (4 wavefronts) covers 4 x 64 output rows-by-columns "cells" of one
//    expert; per item there are ceil(N / (4 slices)) workgroups, so the grid
//    is (items x column groups x K-splits) whatever the shape of the cells.
//  * Wide cells (an expert with a single item, the common case): the 4
//    wavefronts share the item's rows (A tile through LDS) and each streams its
//    own column slice of the weights straight into registers.
//  * Tall cells (runs of 2 items of one expert; a run of 4 is two runs of 2):
//    the wavefronts take different row blocks of the same column slices and
//    share the weight tile through LDS, so such an expert's weights are read
//    once per 128 rows instead of once per 64 rows.
//  * Split-K when the host-side bound on work items is too small to fill the
//    256 CUs (decode-sized batches): each split accumulates a K range into an
//    fp32 partial plane, and a reduce kernel adds the planes in split order
//    and applies the epilogue (SwiGLU, or the router weight).
//  * Matrix cores: v_mfma_f32_16x16x32_{f16,bf16} (v_mfma_f32_16x16x4_f32 for
//    fp32). The weights are row-major [K][N] (N contiguous) but an MFMA lane
//    needs 8 consecutive K of one column. Each lane loads 8 K-rows x 4
//    columns (8-byte loads; 16 lanes cover one 128-byte row segment) and
//    transposes the 8x4 block in registers into 4 B-fragments: fragment c
//    feeds MFMA c, whose 16 columns are the logical columns 4*j + c of the
//    slice. No repacking of the weights by the caller.
//  * Loads of K-step s+S-1 are issued before the MFMAs of step s.
//  * Packed weights (moe_pack_weights, once at load time): each wavefront's
//    K range of a column slice is one contiguous run of 4 KB tiles already in
//    MFMA lane order (16-byte loads, no transposes).
//  * Big cells (packed 16-bit weights, experts with hundreds of rows, as in a
//    long prompt planned as one call): runs of 4 items x 256 weight columns on
//    8 wavefronts, operands loaded straight into LDS (k_big, below), which
//    turns those experts from weight streaming into matrix-core work.
#include "common.hpp"
#include "launch.hpp"
#include "plan_wave.hpp"

namespace moe {

constexpr int kMT = kItemRows / 16;     // 16-row m-tiles per work item
constexpr int kWavesPerBlock = 4;
constexpr int kNpl = 4;                 // columns per lane and B stream
// output columns per 8-wavefront big-cell workgroup: h columns (gate/up) or y
// columns (down)
constexpr int big_cols(bool gateup) { return gateup ? 128 : 256; }

int ffn_rows_per_item() { return kItemRows; }

// Packed weight layout (written once by k_pack, read by the GEMMs with
// PACKED): a matrix [E][Kd][N] becomes, per expert, column group g (4 slices
// of 64*m columns), K-step s, wave slice w and stream m (gate/up: m = 1 stream
// of 64 columns; down: m = 2 halves of 64 columns), a 4 KB tile of 4 x 64
// 16-byte words, word [c][lane] = what MFMA lane `lane` takes as its c-th B
// operand of the step: 16-bit types: the 8 K-values 32s + 8*(lane>>4) + i of
// column (4g+w)*64m + 64*stream + 4*(lane&15) + c; fp32: 4 columns
// (4g+w)*64m + 64*stream + 4*(lane&15) .. +3 of K-row 16s + 4*(lane>>4) + c.
// Outside [0,Kd) x [0,N) the words hold zeros. A workgroup's K range of one
// column group is then one contiguous run of 16 KB (x m) steps.
struct PackedGeom {
    int gs, nst, m;       // column groups, K-steps, streams
    uint32_t step_bytes;  // bytes of one K-step of one column group
};

__host__ __device__ inline PackedGeom packed_geom(int Kd, int N, bool gateup, int es)
{
    PackedGeom z;
    z.m = gateup ? 1 : 2;
    const int kstep = es == 2 ? 32 : 16;
    z.gs = (N + 256 * z.m - 1) / (256 * z.m);
    z.nst = (Kd + kstep - 1) / kstep;
    z.step_bytes = 16384u * (uint32_t)z.m;
    return z;
}

size_t packed_weight_bytes(int E, int Kd, int N, bool gateup, int dtype)
{
    const PackedGeom z = packed_geom(Kd, N, gateup, dtype == 0 ? 4 : 2);
    return (size_t)E * z.gs * z.nst * z.step_bytes;
}

// One 16-byte word of the packed layout per thread (grid-stride); U is the
// raw element (uint16_t for f16/bf16, uint32_t for fp32): bits are copied.
template <typename U>
__global__ __launch_bounds__(256) void k_pack(const U *__restrict__ src, int Kd, int N, int gs,
                                              int nst, int nm, uint4 *__restrict__ dst,
                                              size_t total)
{
    for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (size_t)gridDim.x * 256) {
        const int l = (int)(idx & 63), c = (int)((idx >> 6) & 3);
        size_t t = idx >> 8;
        const int m = (int)(t % nm);
        t /= nm;
        const int w = (int)(t & 3);
        t >>= 2;
        const int s = (int)(t % nst);
        t /= nst;
        const int g = (int)(t % gs);
        const size_t e = t / gs;
        const int n0 = (4 * g + w) * 64 * nm + 64 * m + 4 * (l & 15);
        auto val = [&](int k, int n) -> uint32_t {
            return (k < Kd && n < N) ? (uint32_t)src[(e * Kd + k) * (size_t)N + n] : 0u;
        };
        uint32_t o[4];
        if constexpr (sizeof(U) == 2) {
            const int n = n0 + c, k0 = 32 * s + 8 * (l >> 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = val(k0 + 2 * q, n) | (val(k0 + 2 * q + 1, n) << 16);
        } else {
            const int k = 16 * s + 4 * (l >> 4) + c;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = val(k, n0 + q);
        }
        dst[idx] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

hipError_t launch_pack(int dtype, const void *src, int E, int Kd, int N, bool gateup, void *dst,
                       hipStream_t s)
{
    const PackedGeom z = packed_geom(Kd, N, gateup, dtype == 0 ? 4 : 2);
    const size_t total = (size_t)E * z.gs * z.nst * z.step_bytes / 16;
    const size_t want = (total + 255) / 256;
    const unsigned blocks = (unsigned)(want < (1u << 18) ? want : (1u << 18));
    if (dtype == 0)
        hipLaunchKernelGGL(k_pack<uint32_t>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint32_t *>(src), Kd, N, z.gs, z.nst, z.m,
                           static_cast<uint4 *>(dst), total);
    else
        hipLaunchKernelGGL(k_pack<uint16_t>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const uint16_t *>(src), Kd, N, z.gs, z.nst, z.m,
                           static_cast<uint4 *>(dst), total);
    return hipGetLastError();
}

// Items are ceil(cnt_e / 64) per active expert, so their number is at most
// (active experts) + (entries beyond one per active expert) / 64; with rows
// padded to tm this is bounded from max_rows as below.
int64_t ffn_max_items(int E, int tm, int64_t max_rows)
{
    const int64_t per_tile = (max_rows + tm - 1) / tm;
    return max_rows / kItemRows + 1 + (E < per_tile ? E : per_tile);
}

// A run of 4 items spans more than 3 * 64 rows of one expert.
int64_t ffn_max_quads(int64_t max_rows) { return max_rows / (3 * kItemRows + 1); }

// ---- host-side shape of the two grouped GEMMs ------------------------------
namespace {

// columns of one workgroup's 4 slices: gate/up 4 x 64, down 4 x 128
int group_cols(bool gateup) { return kWavesPerBlock * (gateup ? 16 * kNpl : 32 * kNpl); }

// Split-K is used when the bound on (item, column group) cells is below
// kSplitBelowCells, three quarters of the 256 CUs: then each projection's
// reduction is cut into enough K ranges for about kTargetCells workgroups,
// two per CU. Above it, a split gains less than its reduction launch costs
// (decode, 2,816 x 704 bf16: the down projection's 246 cells unsplit took
// 29.7 us, split in two 27.1 us plus 4.6 us to reduce), while the gate/up
// projection's 123 cells, each streaming 2.9 MB, take 51 us split 5 ways
// (3: 54, 4: 52; 6 ways no longer fits one round of workgroups: 61).
constexpr int64_t kSplitBelowCells = 192;
constexpr int64_t kTargetCells = 512;
// The 8-wavefront kernel takes the runs of 4 items when the plan bound allows
// this many rows per expert on average.
constexpr int64_t kBigMinRowsPerExpert = 64;
constexpr int kMinStepsPerSplit = 8;
constexpr int kMaxSplit = 8;

void split_for(int64_t cells, int Kd, int kstep, int *nsplit, int *steps)
{
    const int nsteps = (Kd + kstep - 1) / kstep;
    int s = 1;
    if (cells < kSplitBelowCells) s = (int)((kTargetCells + cells - 1) / cells);
    s = s < kMaxSplit ? s : kMaxSplit;
    const int smax = nsteps / kMinStepsPerSplit > 1 ? nsteps / kMinStepsPerSplit : 1;
    s = s < smax ? s : smax;
    const int per = (nsteps + s - 1) / s;
    *steps = per;
    *nsplit = (nsteps + per - 1) / per;  // every split has >= 1 step
}

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

FfnShape ffn_shape(int E, int tm, int64_t max_rows, int d, int f, int dtype)
{
    FfnShape z;
    z.max_items = ffn_max_items(E, tm, max_rows);
    z.max_rows = max_rows;
    const int kstep = dtype == 0 ? 16 : 32;
    const int64_t gs_gu = (f + group_cols(true) - 1) / group_cols(true);
    const int64_t gs_dn = (d + group_cols(false) - 1) / group_cols(false);
    split_for(z.max_items * gs_gu, d, kstep, &z.split_gu, &z.steps_gu);
    split_for(z.max_items * gs_dn, f, kstep, &z.split_dn, &z.steps_dn);
    z.blocks_gu = (z.max_items * gs_gu * z.split_gu + 7) / 8 * 8;
    z.blocks_dn = (z.max_items * gs_dn * z.split_dn + 7) / 8 * 8;
    // big cells (packed 16-bit weights, experts with hundreds of rows)
    const bool big = dtype != 0 && max_rows >= kBigMinRowsPerExpert * (int64_t)E;
    z.big_gu = big && z.split_gu == 1;
    z.big_dn = big && z.split_dn == 1;
    z.blocks_big_gu = (ffn_max_quads(max_rows) * ((f + big_cols(true) - 1) / big_cols(true)) + 7) / 8 * 8;
    z.blocks_big_dn = (ffn_max_quads(max_rows) * ((d + big_cols(false) - 1) / big_cols(false)) + 7) / 8 * 8;
    z.plane_gu = max_rows * 2 * (int64_t)f;
    z.plane_dn = max_rows * (int64_t)d;
    const size_t pg = z.split_gu > 1 ? (size_t)z.split_gu * z.plane_gu * 4 : 0;
    const size_t pd = z.split_dn > 1 ? (size_t)z.split_dn * z.plane_dn * 4 : 0;
    z.part_offset = round256(kCtlBytes + (size_t)z.max_items * sizeof(WorkItem));
    z.scratch_bytes = z.part_offset + (pg > pd ? pg : pd);
    return z;
}

// Work list: each expert's row range [eoff[e], eoff[e+1]) cut into items of at
// most kItemRows rows; runs of 4 items first (item_slot). Ranges are clamped
// to [0, max_rows] so that made-up offsets cannot lead outside the buffers.
__global__ __launch_bounds__(1024) void k_worklist(const int32_t *__restrict__ eoff, int E,
                                                   int64_t max_rows, int32_t *__restrict__ ctl,
                                                   WorkItem *__restrict__ items, int max_items,
                                                   int runs_first)
{
    __shared__ int s_q[16], s_r[16], s_p[16];
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
    const int n4 = n & ~3;
    const int qincl = wave_inclusive_scan(n4, lane);
    const int rincl = wave_inclusive_scan(n - n4, lane);
    const int pairs = wave_sum(n - n4 >= 2 ? 2 : 0);  // items in this wave's runs of 2
    if (lane == 63) {
        s_q[wv] = qincl;
        s_r[wv] = rincl;
        s_p[wv] = pairs;
    }
    __syncthreads();
    int qbefore = qincl - n4, rbefore = rincl - (n - n4), qtotal = 0, rtotal = 0, ptotal = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        qbefore += (q < wv) ? s_q[q] : 0;
        rbefore += (q < wv) ? s_r[q] : 0;
        qtotal += s_q[q];
        rtotal += s_r[q];
        ptotal += s_p[q];
    }
    wave_fill_items(n, r0, rows, qbefore, rbefore, qtotal, runs_first != 0, tid, lane, max_items,
                    (int)max_rows, items);
    if (tid == 0) {
        ctl[0] = min(qtotal + rtotal, max_items);
        ctl[1] = runs_first ? min(qtotal, max_items) & ~3 : 0;
        ctl[2] = min(qtotal + ptotal, max_items);
    }
}

// ---- raw buffer loads -----------------------------------------------------
// A buffer resource covering exactly one operand range: loads past its end
// return zeros without touching memory (range-checked by the hardware), which
// zero-fills the K tail of the weights, the rows past a work item's end and
// the steps past the end of a K split.
// Word 3 = 0x00020000: raw (untyped) buffer on gfx9-family GPUs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Cache policy of a buffer load: 0 = default; kNT = non-temporal (the weights
// are read exactly once, so they should not displace the reused row tiles).
constexpr int kNT = 2;

// s_waitcnt vmcnt(n), expcnt and lgkmcnt left at their maximum (no wait)
constexpr int wait_vm(int n) { return 0x0F70 | n; }

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
__device__ __forceinline__ void store_nt(uint4 *p, uint4 v)
{
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u4{v.x, v.y, v.z, v.w}, reinterpret_cast<u4 *>(p));
}

// Stores of the down projection's y, which the combine reads next: buffer
// stores with cache policy sc1 only. Measured on the prefill layer against
// non-temporal stores: the down projection ~15 us and the combine ~7 us faster
// (its y reads then hit the Infinity Cache). Default-policy stores were slower
// than both, and sc1 stores of the gate/up output h gained nothing.
constexpr int kSC1 = 16;
template <int POLICY = kSC1>
__device__ __forceinline__ void store_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v)
{
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off, 0, POLICY);
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

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp) in
// place of an IEEE division: an order of magnitude below the error of the
// fp16/bf16 SwiGLU output it feeds, and a fraction of the epilogue's time
__device__ __forceinline__ float silu(float z)
{
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// 16-bit B operand: RP consecutive K-rows of 4 columns each (row i = K-value
// i). Column c of them as RP/2 words of an MFMA operand (element i = K-row i).
template <int RP>
__device__ __forceinline__ void column_of_rows(const uint2 (&r)[RP], int c, uint32_t (&o)[RP / 2])
{
#pragma unroll
    for (int p = 0; p < RP / 2; ++p) {
        const uint32_t lo = (c < 2) ? r[2 * p].x : r[2 * p].y;
        const uint32_t hi = (c < 2) ? r[2 * p + 1].x : r[2 * p + 1].y;
        o[p] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
}

__device__ __forceinline__ uint4 column_of_rows(const uint2 (&r)[8], int c)
{
    uint32_t o[4];
    column_of_rows<8>(r, c, o);
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

__device__ __forceinline__ uint4 mask4(uint4 v, uint32_t m)
{
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Arguments of one grouped GEMM launch.
//   gate/up: A = xs [rows][d] (or x [a_rows][d] when GATHERED), B0 = W_gate,
//            B1 = W_up [E][d][f], out = h [rows][f] (type T).
//   down:    A = h [rows][f], B0 = W_down [E][f][d], out = y [rows][d] (fp32),
//            stok / sw for the epilogue.
// With nsplit > 1 the epilogue instead writes fp32 partial sums: split s at
// part + s * plane, row r at r * 2N (gate: columns [0, N), up: [N, 2N)) or at
// r * N (down, without the router weight).
// The item count and the work items are separate __restrict__ kernel
// arguments: provably read-only, they are fetched with scalar loads.
struct GemmArgs {
    const void *A;
    const void *B0;
    const void *B1;
    const int32_t *stok;
    const float *sw;
    void *out;
    float *part;
    int64_t plane;
    int a_rows;
    int Kd, N;
    int nsplit;       // K splits per (item, column group)
    int split_steps;  // K-steps per split
    int skip_quads;   // 1: the items in runs of 4 (the first ctl[1]) are left to k_big
    // down projection, compact outputs: out holds binary16 rows and yexp their
    // exponents, block-major: yexp[b * estride + row] for the kY16Block columns
    // of block b (estride = max_rows); nullptr: fp32 y
    int8_t *yexp;
    int64_t estride;
};

__device__ __forceinline__ void store_b64(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v,
                                          int policy_sc1)
{
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    if (policy_sc1)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, v), r, off, 0, kSC1);
    else
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, v), r, off, 0, kNT);
}

// One row of a down cell in the compact format. This lane holds the row's
// values v[m][c] at columns col + m * 64 + c; the 16 lanes of its DPP row hold
// the row's columns [col0, col0 + 128), one exponent block. Lanes whose
// columns lie past N contribute nothing and store nothing, but take part in
// the row maximum (every lane of the row must be active here). ry covers the
// item's rows of binary16 y; rl is the row within the item. Stores: sc1
// (policy_sc1) or non-temporal. Returns the row's exponent (the same in all
// 16 lanes); the caller stores the exponents (store_y16_exponents).
__device__ __forceinline__ int store_y16_row(const GemmArgs &p, __amdgpu_buffer_rsrc_t ry, int rl,
                                             int col, const float (&v)[2][4], int policy_sc1)
{
    constexpr int HALF = 16 * kNpl;
    const int N = p.N;
    float M = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            M = __builtin_fmaxf(M, col + m * HALF < N ? __builtin_fabsf(v[m][c]) : 0.0f);
    const int e = y16_exponent(row16_fmax(M));
    const float scale = pow2f(e);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        if (col + m * HALF >= N) continue;
        float q[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) q[c] = v[m][c] * scale;
        store_b64(ry, (uint32_t)((rl * N + col + m * HALF) * 2),
                  make_uint2(Elt<_Float16>::pack2(q[0], q[1]), Elt<_Float16>::pack2(q[2], q[3])),
                  policy_sc1);
    }
    return e;
}

// The exponents of a wavefront's 64 rows of one block, in one store: ev[mt][r]
// is the exponent of row 16 mt + 4 kg + r (kg = the lane's DPP row), so lane
// (kg, nq) already holds row 16 (nq >> 2) + 4 kg + (nq & 3) -- the 64 lanes
// hold the 64 rows once each -- and stores it if `real` (its row holds an
// entry). yexp_block = the block's exponents, row0 = the item's first row.
template <int NMT>
__device__ __forceinline__ void store_y16_exponents(int8_t *yexp_block, int64_t row0,
                                                    const int (&ev)[NMT][4], int rl, bool real)
{
    const int nq = threadIdx.x & 15;
    int e = 0;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) e = (mt == (nq >> 2) && r == (nq & 3)) ? ev[mt][r] : e;
    if (real) yexp_block[row0 + rl] = (int8_t)e;
}

// Epilogue of one wavefront: acc[m][mt][c][r] is the output at row
// 16*mt + 4*kg + r of item `it` and column col + c (+ HALF for m = 1 of the
// down projection). rinfo[l] = (router weight, token) of the item's row l.
template <typename T, bool GATEUP, int NMT, bool MAY_SPLIT = true>
__device__ __forceinline__ void store_cells(const GemmArgs &p, const WorkItem &it, int col, int kg,
                                            const float4_t (&acc)[2][NMT][kNpl],
                                            const float2 *__restrict__ rinfo, int split)
{
    constexpr int ES = sizeof(T);
    constexpr int HALF = GATEUP ? 0 : 16 * kNpl;
    const int N = p.N;
    const bool partial = MAY_SPLIT && p.nsplit > 1;
    if constexpr (!GATEUP && ES == 2) {
        if (p.yexp && !partial) {
            // compact y: every lane stays for the row maxima (no early exit by column)
            const int col0 = col - kNpl * (threadIdx.x & 15);
            if (col0 >= N) return;  // the whole slice lies past N (wave-uniform)
            const __amdgpu_buffer_rsrc_t ry =
                make_rsrc(static_cast<uint16_t *>(p.out) + (int64_t)it.row0 * N,
                          (uint32_t)(it.nrows * N * 2));
            int ev[NMT][4];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ev[mt][r] = 0;
                    const int rl = 16 * mt + 4 * kg + r;
                    if (rl >= it.nrows) continue;  // uniform over the DPP row
                    const float2 ri = rinfo[rl];
                    if (__float_as_int(ri.y) < 0) continue;  // pad rows are never combined
                    float v[2][4];
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int c = 0; c < 4; ++c) v[m][c] = ri.x * acc[m][mt][c][r];
                    ev[mt][r] = store_y16_row(p, ry, rl, col, v, 1);
                }
            const int nq = threadIdx.x & 15;
            const int rl = 16 * (nq >> 2) + 4 * kg + (nq & 3);
            const bool real = rl < it.nrows && __float_as_int(rinfo[rl].y) >= 0;
            store_y16_exponents<NMT>(p.yexp + (col0 / kY16Block) * p.estride, it.row0, ev, rl,
                                     real);
            return;
        }
    }
    if (col >= N) return;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = 16 * mt + 4 * kg + r;
            if (rl >= it.nrows) continue;
            const int64_t row = it.row0 + rl;
            if constexpr (GATEUP) {
                if (partial) {
                    // pad rows: the reduction writes their zero h without reading
                    if (__float_as_int(rinfo[rl].y) < 0) continue;
                    float *P = p.part + split * p.plane + row * 2 * N + col;
#pragma unroll
                    for (int m = 0; m < 2; ++m)
                        *reinterpret_cast<float4 *>(P + m * N) =
                            make_float4(acc[m][mt][0][r], acc[m][mt][1][r], acc[m][mt][2][r],
                                        acc[m][mt][3][r]);
                    continue;
                }
                float hv[kNpl];
#pragma unroll
                for (int c = 0; c < kNpl; ++c) hv[c] = silu(acc[0][mt][c][r]) * acc[1][mt][c][r];
                T *H = static_cast<T *>(p.out) + row * N + col;
                if constexpr (ES == 2)
                    store_nt(reinterpret_cast<uint2 *>(H),
                             make_uint2(Elt<T>::pack2(hv[0], hv[1]), Elt<T>::pack2(hv[2], hv[3])));
                else
                    store_nt(reinterpret_cast<float4 *>(H), make_float4(hv[0], hv[1], hv[2], hv[3]));
            } else {
                const float2 ri = rinfo[rl];
                if (__float_as_int(ri.y) < 0) continue;  // pad rows are never combined
                const float g = partial ? 1.0f : ri.x;
                float *P = p.part + split * p.plane + row * N + col;
                // the item's rows of y, as one descriptor (range-checked stores)
                const __amdgpu_buffer_rsrc_t ry =
                    make_rsrc(static_cast<float *>(p.out) + (int64_t)it.row0 * N,
                              (uint32_t)(it.nrows * N * 4));
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (col + m * HALF >= N) continue;
                    const float4 v = make_float4(g * acc[m][mt][0][r], g * acc[m][mt][1][r],
                                                 g * acc[m][mt][2][r], g * acc[m][mt][3][r]);
                    if (partial)
                        *reinterpret_cast<float4 *>(P + m * HALF) = v;
                    else
                        store_sc1(ry, (uint32_t)((rl * N + col + m * HALF) * 4), v);
                }
            }
        }
    }
}

// (router weight, token) of the item's rows for the epilogue; the gate/up
// projection has no router weight (sw is not passed) and needs the tokens only
// (ltok != nullptr: the item's tokens from LDS, ltok[l] for its row l)
template <bool WITH_SW>
__device__ __forceinline__ void load_rinfo(const GemmArgs &p, const WorkItem &it, int l,
                                           float2 *__restrict__ rinfo, const int *ltok = nullptr)
{
    const bool ok = l < it.nrows;
    const int64_t r = it.row0 + (ok ? l : 0);
    const int t = ok ? (ltok ? ltok[l] : p.stok[r]) : -1;
    rinfo[l] = make_float2(WITH_SW && ok ? p.sw[r] : 0.f, __int_as_float(t));
}

// Launches with fewer cells than this (the GPU's workgroup slots: 2 per CU)
// stream their weights deep (see wide_cells)
constexpr int kDeepBelowCells = 512;

// Pipeline depth of the wide cells for NMT m-tiles: stage = 32 B-operand + 4
// A-operand VGPRs, accumulators = 32*NMT VGPRs; S stages + accumulators stay
// <= ~232.
constexpr int stages_for(int nmt) { return nmt >= 4 ? 2 : nmt == 3 ? 3 : nmt == 2 ? 4 : 5; }

// Shared A tile of one K-step: 64 rows x 32 K (16-bit) or 64 rows x 16 K
// (fp32), 64 bytes per row, double-buffered: 2 x 4 KB of LDS per workgroup.
constexpr int kATileU4 = kItemRows * 64 / 16;
// Shared B tile of the tall cells: per column slice 2 matrices x 64 lanes x
// 64 bytes (4 fragments of 16 bytes per lane), double-buffered.
constexpr int tall_buf_u4(int nslices) { return nslices * 2 * 64 * 4; }
constexpr int kLdsU4 = 2 * tall_buf_u4(2) > 2 * kATileU4 ? 2 * tall_buf_u4(2) : 2 * kATileU4;

// Wide cells: a workgroup of 4 wavefronts computes one work item (<= 64 rows)
// against 4 adjacent column slices of 16*kNpl columns, one per wavefront.
//  * A (the item's rows) is shared: per K-step each wavefront loads 16 rows x
//    64 bytes (one 16-byte load per lane) into registers, writes them to an LDS
//    slot, and after one barrier every wavefront reads its MFMA A-fragments
//    from LDS. One copy of A per workgroup instead of one per wavefront.
//  * B (the weights) is private to each wavefront: lane l supplies MFMA column
//    (l & 15) and K-group (l >> 4); it loads KR K-rows x kNpl columns of each
//    weight matrix per step (16 lanes cover one 16*kNpl-column row segment) and
//    transposes them in registers, so MFMA c produces the logical columns
//    kNpl*j + c, j = 0..15.
//  * S-stage register ring: the loads of step s+S-1 are issued before the
//    MFMAs of step s; the loop body is straight-line code, so they stay in
//    flight. The per-step barrier keeps the 4 wavefronts in step, so together
//    they read 4 adjacent row segments of every weight row.
//  * depth of the weight stream, one policy per launch (ctl[2]): when most
//    items are single (each streams its expert's weights from HBM once) the
//    launch runs shallow: the row operand's K-tail mask is applied as it is
//    loaded, so a wavefront waits for the step it has just issued (all but
//    its last few loads) before computing, about one step per wavefront in
//    flight. More only queues in the memory system: on a 2,048-token prefill
//    layer (512 experts, single items) masking at the use, with S-1 steps in
//    flight, was 4% slower. When most items are in runs (skewed routing; the
//    runs' tiles are re-read from L2) the mask moves to the use and the ring
//    keeps S-1 steps in flight: 7% faster on the down projection of a skewed
//    2,048-token chunk. Shallow single items beside deep runs in one launch
//    measured slower than either policy. A launch of fewer cells than the GPU
//    holds at once (kDeepBelowCells, two per CU) runs deep too: no other
//    workgroup shares a CU's memory pipe, so a workgroup's own bytes in flight
//    set its rate (decode's down projection, 186 cells: 30.3 -> 25.1 us).
// GATHERED (gate/up only): A is the token activation x [a_rows][Kd] and row r
// of the item reads x[stok[r]] -- the gather fused into the A-tile loads.
// The K range is [kb, ke) (a split of the reduction, or all of it).
template <typename T, bool GATEUP, bool GATHERED, bool PACKED, bool DEEP, int NMT>
__device__ __forceinline__ void wide_cells(const GemmArgs &p, const WorkItem it, int slice,
                                           int kb, int ke, int split, uint4 *__restrict__ a_lds,
                                           float2 *__restrict__ rinfo, const int *ltok)
{
    constexpr int NPL = kNpl;
    constexpr int ES = sizeof(T);
    constexpr int KR = Elt<T>::KR;
    constexpr int KSTEP = 4 * KR;
    constexpr int NMAT = 2;       // two B streams (see below)
    constexpr int LB = NPL * ES;  // bytes per lane per row
    const T *A = static_cast<const T *>(p.A);
    const T *B0 = static_cast<const T *>(p.B0);
    const T *B1 = static_cast<const T *>(p.B1);
    const int Kd = p.Kd, N = p.N;

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

    // operand ranges: this expert's weight rows [kb, ke) (empty for a surplus
    // slice: its loads return zeros without memory traffic), this item's rows
    __amdgpu_buffer_rsrc_t rb0, rb1;
    uint32_t vcol, rowb, bstep;  // lane offset, B row stride, B bytes per K-step
    if constexpr (PACKED) {
        // this wavefront's tiles (g, s, w, m) for s in [s0, s1): 4 KB each,
        // one K-step apart (16 KB x streams)
        const int g = slice >> 2, w = slice & 3;
        const PackedGeom z = packed_geom(Kd, N, GATEUP, ES);
        const int s0 = kb / KSTEP, s1 = (ke + KSTEP - 1) / KSTEP;
        const size_t tb = ((((size_t)it.expert * z.gs + g) * z.nst + s0) * 4 + w) * z.m * 4096;
        const uint32_t span = (uint32_t)(s1 - s0) * z.step_bytes;
        const uint32_t r0 = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(slice_ok ? span - (uint32_t)(w * z.m) * 4096u : 0u));
        const uint32_t r1 = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(slice_ok ? span - (uint32_t)(w * z.m + z.m - 1) * 4096u : 0u));
        const char *b0c = static_cast<const char *>(p.B0);
        rb0 = make_rsrc(b0c + tb, r0);
        rb1 = GATEUP ? make_rsrc(static_cast<const char *>(p.B1) + tb, r0)
                     : make_rsrc(b0c + tb + 4096, r1);
        vcol = (uint32_t)lane * 16;
        rowb = 1024;  // between fragments c of one lane
        bstep = z.step_bytes;
    } else {
        const size_t wofs = (size_t)it.expert * Kd * N + (size_t)kb * N;
        const uint32_t kbytes = (uint32_t)((size_t)(ke - kb) * N * ES);
        const uint32_t wbytes = slice_ok ? kbytes : 0u;
        rb0 = make_rsrc(B0 + wofs, wbytes);
        // ((ke-kb)*N >= 8*8 >= HALF, so the second range never underflows;
        // readfirstlane keeps the wave-uniform value in an SGPR)
        const uint32_t wbytes1 = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(slice_ok ? kbytes - (uint32_t)(HALF * ES) : 0u));
        rb1 = GATEUP ? make_rsrc(B1 + wofs, wbytes) : make_rsrc(B0 + wofs + HALF, wbytes1);
        rowb = (uint32_t)N * ES;  // bytes per weight row
        vcol = (uint32_t)col * ES;
        bstep = (uint32_t)KSTEP * rowb;
    }
    // this thread's share of the A tile: row tid/4, 16-byte chunk tid%4
    const int arow = tid >> 2, achunk = (tid & 3) * (16 / ES);
    __amdgpu_buffer_rsrc_t ra;
    uint32_t va0;
    if constexpr (GATHERED) {
        // all of x (< 2 GiB, checked by the host); a pad row (token -1) or a
        // row past the item starts at 2^31, outside the range: it reads zeros
        ra = make_rsrc(A, (uint32_t)((size_t)p.a_rows * Kd * ES));
        const int t = arow < it.nrows ? (ltok ? ltok[arow] : p.stok[it.row0 + arow]) : -1;
        va0 = (unsigned)t < (unsigned)p.a_rows ? (uint32_t)t * (uint32_t)Kd * ES : 0x80000000u;
    } else {
        ra = make_rsrc(A + (size_t)it.row0 * Kd, (uint32_t)((size_t)it.nrows * Kd * ES));
        va0 = (uint32_t)arow * (uint32_t)Kd * ES;
    }

    // made visible to all wavefronts by the barriers of the K loop (gate/up
    // needs the tokens only for its partial sums)
    if (!GATEUP || p.nsplit > 1)
        if (tid < kItemRows) load_rinfo<!GATEUP>(p, it, tid, rinfo, ltok);

    float4_t acc[NMAT][NMT][NPL];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int c = 0; c < NPL; ++c) acc[m][mt][c] = float4_t{0.f, 0.f, 0.f, 0.f};

    // packed: 4 fragments (fp32: 4 rows) of 16 bytes per stream and step
    constexpr int NB = PACKED ? 4 : KR;
    constexpr int LBB = PACKED ? 16 : LB;
    typedef typename Ld<LBB>::type BT;
    struct Stage {
        BT b[NMAT][NB];
        uint4 a;
    };
    auto load = [&](Stage &st, int k0) {
        const uint32_t vb = PACKED ? vcol + (uint32_t)((k0 - kb) / KSTEP) * bstep
                                   : vcol + (uint32_t)(k0 + KR * kg - kb) * rowb;
#pragma unroll
        for (int i = 0; i < NB; ++i) st.b[0][i] = Ld<LBB, kNT>::run(rb0, vb, (uint32_t)i * rowb);
#pragma unroll
        for (int i = 0; i < NB; ++i) st.b[1][i] = Ld<LBB, kNT>::run(rb1, vb, (uint32_t)i * rowb);
        // K past the range: the weights read as zero; zero A too so that no
        // non-finite value of a neighbouring row can leak in as 0 * inf.
        // Shallow: masked here, which makes the wavefront wait for the step's
        // loads right after issuing them; deep: masked at its use
        const int ka = k0 + achunk;
        st.a = Ld<16>::run(ra, va0 + (uint32_t)ka * ES, 0u);
        if constexpr (!DEEP) st.a = mask4(st.a, ka < ke ? 0xffffffffu : 0u);
    };
    auto compute = [&](const Stage &st, int step) {
        uint4 *slot = a_lds + (step & 1) * kATileU4;
        const int ka = kb + step * KSTEP + achunk;
        slot[tid] = DEEP ? mask4(st.a, ka < ke ? 0xffffffffu : 0u) : st.a;
        __syncthreads();
        uint4 af[NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) af[mt] = slot[(16 * mt + nq) * 4 + kg];
        if constexpr (ES == 2) {
#pragma unroll
            for (int c = 0; c < NPL; ++c) {
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    uint4 fb;
                    if constexpr (PACKED)
                        fb = st.b[m][c];
                    else
                        fb = column_of_rows(st.b[m], c);
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
    const int nsteps = (ke - kb + KSTEP - 1) / KSTEP;
    Stage st[S];
    // deep: the prologue's loads stay in step order (the load-count waits at
    // the loop head are taken over both entries into it)
#pragma unroll
    for (int j = 0; j < S - 1; ++j) {
        load(st[j], kb + j * KSTEP);
        if constexpr (DEEP) __builtin_amdgcn_sched_barrier(0);
    }
    for (int s = 0; s < nsteps; s += S) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            // steps past the range load zero weights (no memory traffic) and add 0
            load(st[(j + S - 1) % S], kb + (s + j + S - 1) * KSTEP);
            __builtin_amdgcn_sched_barrier(0);
            compute(st[j], s + j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    store_cells<T, GATEUP, NMT>(p, it, col, kg, acc, rinfo, split);
}

// Tall cells: a run of R consecutive items of one expert (R = 2 is dispatched;
// the R = 4 shape, one column slice over 256 rows, measured slower). The 4
// wavefronts take row block rb = wave % R (item i0 + rb, 64 rows) and column
// slice cs = wave / R of the C = 4/R slices of the workgroup, so the C
// slices' weight tile is loaded once per K-step and shared through LDS by R
// wavefronts each:
//  * producers: the 256 threads split the tile into units of (slice, matrix,
//    MFMA lane); a thread loads RP = KR*C/2 K-rows x 4 columns of its unit,
//    transposes them in registers (16-bit) and writes the MFMA B fragments of
//    that lane to LDS;
//  * consumers: every wavefront reads its slice's fragments from LDS and its
//    own rows' A fragments straight from memory (16-byte loads per lane).
// Every wavefront computes 4 m-tiles (a short last item computes zero rows).
// The weight loads keep the default cache policy here: the other runs of the
// same expert read the same tile, often while it is still in L2.
template <typename T, bool GATEUP, bool GATHERED, bool PACKED, bool DEEP, int R>
__device__ __forceinline__ void tall_cells(const GemmArgs &p, const WorkItem *__restrict__ items,
                                           int i0, int nitems, int g, int j, int kb, int ke,
                                           int split, uint4 *__restrict__ lds,
                                           float2 *__restrict__ rinfo)
{
    constexpr int NPL = kNpl;
    constexpr int ES = sizeof(T);
    constexpr int KR = Elt<T>::KR;
    constexpr int KSTEP = 4 * KR;
    constexpr int NMAT = 2;
    constexpr int NMT = kMT;
    constexpr int C = 4 / R;    // column slices per workgroup
    constexpr int H = 2 / C;    // producer threads per (slice, matrix, lane) unit
    constexpr int RP = KR / H;  // weight rows per producer thread
    constexpr int SW = GATEUP ? 16 * NPL : 32 * NPL;
    constexpr int HALF = GATEUP ? 0 : 16 * NPL;
    constexpr int LB = NPL * ES;
    constexpr int BUF = tall_buf_u4(C);
    static_assert(H * C == 2 && RP * H == KR, "tall cell shape");
    const T *A = static_cast<const T *>(p.A);
    const T *B0 = static_cast<const T *>(p.B0);
    const T *B1 = static_cast<const T *>(p.B1);
    const int Kd = p.Kd, N = p.N;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nq = lane & 15, kg = lane >> 4;

    // consumer role: item i0 + rb of the run, column slice cs
    const int rb = wave % R, cs = wave / R;
    const WorkItem first = items[i0];
    const int expert = first.expert;
    WorkItem it = first;
    if (rb != 0) {
        if (i0 + rb < nitems) it = items[i0 + rb];
        if (i0 + rb >= nitems || it.expert != expert) it.nrows = 0;
    }
    const int col = (4 * g + C * j + cs) * SW + NPL * nq;

    // producer role: unit (slice pcs, matrix pm, lane plu), rows RP*hh.. of it
    const int pcs = C == 1 ? 0 : (wave >> 1);
    const int pm = C == 1 ? (wave >> 1) : (wave & 1);
    const int plu = C == 1 ? ((tid >> 1) & 63) : lane;
    const int hh = C == 1 ? (tid & 1) : 0;
    const int pslice = 4 * g + C * j + pcs;
    // packed: a producer thread copies 4/H whole fragments (fp32: rows) of its unit
    constexpr int PNB = PACKED ? 4 / H : RP;
    __amdgpu_buffer_rsrc_t rbp;
    uint32_t rowb, vpb, bstep;
    if constexpr (PACKED) {
        const PackedGeom z = packed_geom(Kd, N, GATEUP, ES);
        const int s0 = kb / KSTEP, s1 = (ke + KSTEP - 1) / KSTEP;
        const int wp = C * j + pcs, mm = GATEUP ? 0 : pm;  // tile slot in the group
        const size_t tb =
            (((((size_t)expert * z.gs + g) * z.nst + s0) * 4 + wp) * z.m + mm) * 4096;
        const uint32_t span = (uint32_t)(s1 - s0) * z.step_bytes;
        const uint32_t pbytes = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(pslice * SW >= N ? 0u : span - (uint32_t)(wp * z.m + mm) * 4096u));
        const char *bb = static_cast<const char *>(GATEUP && pm ? p.B1 : p.B0);
        rbp = make_rsrc(bb + tb, pbytes);
        rowb = 1024;
        vpb = (uint32_t)(hh * PNB) * 1024 + (uint32_t)plu * 16;
        bstep = z.step_bytes;
    } else {
        const size_t wofs = (size_t)expert * Kd * N + (size_t)kb * N;
        const uint32_t kbytes = (uint32_t)((size_t)(ke - kb) * N * ES);
        // pm and pslice are wave-uniform: keep the range and base in SGPRs
        const uint32_t pbytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)(
            pslice * SW >= N ? 0u
                             : (GATEUP || pm == 0) ? kbytes : kbytes - (uint32_t)(HALF * ES)));
        const T *pbase = GATEUP ? (pm ? B1 + wofs : B0 + wofs) : B0 + wofs + pm * HALF;
        rbp = make_rsrc(pbase, pbytes);
        rowb = (uint32_t)N * ES;
        vpb = (uint32_t)(pslice * SW + NPL * (plu & 15)) * ES +
              (uint32_t)(KR * (plu >> 4) + RP * hh) * rowb;
        bstep = (uint32_t)KSTEP * rowb;
    }

    // A: 4 m-tiles of this wavefront's item; lane row 16*mt + nq, K chunk kg
    __amdgpu_buffer_rsrc_t ra;
    uint32_t va[NMT];
    if constexpr (GATHERED) {
        ra = make_rsrc(A, (uint32_t)((size_t)p.a_rows * Kd * ES));
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            const int rl = 16 * mt + nq;
            const int t = rl < it.nrows ? p.stok[it.row0 + rl] : -1;
            va[mt] = (unsigned)t < (unsigned)p.a_rows ? (uint32_t)t * (uint32_t)Kd * ES : 0x80000000u;
        }
    } else {
        ra = make_rsrc(A + (size_t)it.row0 * Kd, (uint32_t)((size_t)it.nrows * Kd * ES));
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) va[mt] = (uint32_t)(16 * mt + nq) * (uint32_t)Kd * ES;
    }

    float2 *my_rinfo = rinfo + wave * kItemRows;
    if (!GATEUP || p.nsplit > 1) load_rinfo<!GATEUP>(p, it, lane, my_rinfo);

    float4_t acc[NMAT][NMT][NPL];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int c = 0; c < NPL; ++c) acc[m][mt][c] = float4_t{0.f, 0.f, 0.f, 0.f};

    constexpr int LBB = PACKED ? 16 : LB;
    typedef typename Ld<LBB>::type BT;
    struct Stage {
        BT b[PNB];
        uint4 a[NMT];
    };
    auto load = [&](Stage &st, int k0) {
        const uint32_t vb = vpb + (uint32_t)((k0 - kb) / KSTEP) * bstep;
#pragma unroll
        for (int i = 0; i < PNB; ++i) st.b[i] = Ld<LBB>::run(rbp, vb, (uint32_t)i * rowb);
        // A past the K range masked here (shallow) or at its use (deep), as in
        // the wide cells
        const int ka = k0 + KR * kg;
        const uint32_t am = ka < ke ? 0xffffffffu : 0u;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            st.a[mt] = Ld<16>::run(ra, va[mt] + (uint32_t)ka * ES, 0u);
            if constexpr (!DEEP) st.a[mt] = mask4(st.a[mt], am);
        }
    };
    // fragment (or fp32 row) q of lane l of slice s, matrix m in a buffer
    auto frag = [&](int s, int m, int q, int l) { return ((s * NMAT + m) * 4 + q) * 64 + l; };
    auto compute = [&](const Stage &st, int step) {
        uint4 *buf = lds + (step & 1) * BUF;
        const uint32_t am = kb + step * KSTEP + KR * kg < ke ? 0xffffffffu : 0u;
        uint4 a[NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) a[mt] = DEEP ? mask4(st.a[mt], am) : st.a[mt];
        if constexpr (PACKED) {
#pragma unroll
            for (int i = 0; i < PNB; ++i) buf[frag(pcs, pm, PNB * hh + i, plu)] = st.b[i];
        } else if constexpr (ES == 2) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint32_t o[RP / 2];
                column_of_rows<RP>(st.b, c, o);
                if constexpr (RP == 8)
                    buf[frag(pcs, pm, c, plu)] = make_uint4(o[0], o[1], o[2], o[3]);
                else
                    reinterpret_cast<uint2 *>(buf)[2 * frag(pcs, pm, c, plu) + hh] =
                        make_uint2(o[0], o[1]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < RP; ++i) buf[frag(pcs, pm, RP * hh + i, plu)] = st.b[i];
        }
        __syncthreads();
        if constexpr (ES == 2) {
#pragma unroll
            for (int c = 0; c < NPL; ++c)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    const uint4 fb = buf[frag(cs, m, c, lane)];
#pragma unroll
                    for (int mt = 0; mt < NMT; ++mt)
                        acc[m][mt][c] = Elt<T>::mfma(a[mt], fb, acc[m][mt][c]);
                }
        } else {
#pragma unroll
            for (int q = 0; q < KR; ++q)
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    const uint4 bq = buf[frag(cs, m, q, lane)];
#pragma unroll
                    for (int c = 0; c < NPL; ++c)
#pragma unroll
                        for (int mt = 0; mt < NMT; ++mt)
                            acc[m][mt][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                lanef(a[mt], q), lanef(bq, c), acc[m][mt][c], 0, 0, 0);
                }
        }
    };

    // register ring depth: 16-bit 4 (one slice) or 3 (two slices) stages;
    // fp32 stages are larger, 2
    constexpr int S = ES == 2 ? (C == 1 ? 4 : 3) : 2;
    const int nsteps = (ke - kb + KSTEP - 1) / KSTEP;
    Stage st[S];
#pragma unroll
    for (int jj = 0; jj < S - 1; ++jj) {  // as in the wide cells
        load(st[jj], kb + jj * KSTEP);
        if constexpr (DEEP) __builtin_amdgcn_sched_barrier(0);
    }
    for (int s = 0; s < nsteps; s += S) {
#pragma unroll
        for (int jj = 0; jj < S; ++jj) {
            load(st[(jj + S - 1) % S], kb + (s + jj + S - 1) * KSTEP);
            __builtin_amdgcn_sched_barrier(0);
            compute(st[jj], s + jj);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    store_cells<T, GATEUP, NMT>(p, it, col, kg, acc, my_rinfo, split);
}

// The cell of item i: a tall cell for an item in a run, else a wide cell.
template <typename T, bool GATEUP, bool GATHERED, bool PACKED, bool DEEP>
__device__ __forceinline__ void gemm_cell(const GemmArgs &p, const WorkItem *__restrict__ items,
                                          const WorkItem it, int i, int nitems, int g, int kb,
                                          int ke, int split, uint4 *__restrict__ lds,
                                          float2 *__restrict__ rinfo)
{
    const int run = it.run & 0xff, j = (it.run >> 8) & 0xff;
    // a run of 4 is taken as two runs of 2 (4-item cells, one column slice of
    // 256 rows each: the skewed long prompt's layer 0.8% slower)
    if (run == 4 && j < 4 && i >= j) {
        tall_cells<T, GATEUP, GATHERED, PACKED, DEEP, 2>(p, items, i - (j & 1), nitems, g, j & 1,
                                                         kb, ke, split, lds, rinfo);
        return;
    }
    if (run == 2 && j < 2 && i >= j) {
        tall_cells<T, GATEUP, GATHERED, PACKED, DEEP, 2>(p, items, i - j, nitems, g, j, kb, ke,
                                                         split, lds, rinfo);
        return;
    }
    // wave-uniform by construction, so the buffer descriptors live in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = g * kWavesPerBlock + wave;
    switch ((it.nrows + 15) >> 4) {  // m-tiles of this item (uniform per workgroup)
    case 1: wide_cells<T, GATEUP, GATHERED, PACKED, DEEP, 1>(p, it, slice, kb, ke, split, lds, rinfo, nullptr); break;
    case 2: wide_cells<T, GATEUP, GATHERED, PACKED, DEEP, 2>(p, it, slice, kb, ke, split, lds, rinfo, nullptr); break;
    case 3: wide_cells<T, GATEUP, GATHERED, PACKED, DEEP, 3>(p, it, slice, kb, ke, split, lds, rinfo, nullptr); break;
    default: wide_cells<T, GATEUP, GATHERED, PACKED, DEEP, kMT>(p, it, slice, kb, ke, split, lds, rinfo, nullptr); break;
    }
}

// A single item's wide cell, its token rows from LDS (ltok[r] for row r).
template <typename T, bool GATEUP, bool GATHERED, bool PACKED, bool DEEP>
__device__ __forceinline__ void single_cell(const GemmArgs &p, const WorkItem it, int g, int kb,
                                            int ke, int split, uint4 *__restrict__ lds,
                                            float2 *__restrict__ rinfo, const int *ltok)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = g * kWavesPerBlock + wave;
    switch ((it.nrows + 15) >> 4) {  // m-tiles of this item (uniform per workgroup)
    case 1: wide_cells<T, GATEUP, GATHERED, PACKED, DEEP, 1>(p, it, slice, kb, ke, split, lds, rinfo, ltok); break;
    case 2: wide_cells<T, GATEUP, GATHERED, PACKED, DEEP, 2>(p, it, slice, kb, ke, split, lds, rinfo, ltok); break;
    case 3: wide_cells<T, GATEUP, GATHERED, PACKED, DEEP, 3>(p, it, slice, kb, ke, split, lds, rinfo, ltok); break;
    default: wide_cells<T, GATEUP, GATHERED, PACKED, DEEP, kMT>(p, it, slice, kb, ke, split, lds, rinfo, ltok); break;
    }
}

// One workgroup per (work item, group of 4 column slices, K split).
// WP (gathered gate/up of a call planned here, WavePlan wp): workgroup 0
// writes the plan and the work list for the later kernels (plan_wave_body,
// one wavefront, LDS borrowed from the tiles), workgroups 1-7 have nothing
// to do, and workgroup 8 + b finds the item of its logical block b from the
// ids (wave_plan_item: every item is single, so there are no runs and no list
// to read) and keeps the item's tokens in LDS for its A-operand rows. A
// template instance of its own, so that the other launches' code is
// untouched.
template <typename T, bool GATEUP, bool GATHERED, bool PACKED, bool WP = false>
__global__ __launch_bounds__(256, 2) void k_expert_gemm(const GemmArgs p,
                                                        const int32_t *__restrict__ ctl,
                                                        const WorkItem *__restrict__ items,
                                                        const WavePlan wp)
{
    __shared__ uint4 lds[kLdsU4];
    __shared__ float2 rinfo[kWavesPerBlock * kItemRows];
    constexpr int SW = GATEUP ? 16 * kNpl : 32 * kNpl;  // columns per slice
    constexpr int KSTEP = 4 * Elt<T>::KR;
    const int gs = (p.N + 4 * SW - 1) / (4 * SW);       // column groups per item
    const int per_item = gs * p.nsplit;
    if constexpr (WP) {
        static_assert(GATEUP && GATHERED, "planned here: the gathered gate/up launch only");
        static_assert(2 * kMaxExperts * 4 <= kLdsU4 * 16, "plan counters fit the tile LDS");
        __shared__ int s_tok[kItemRows];
        __shared__ WorkItem s_item;
        __shared__ int s_nb[2];
        if (blockIdx.x < 8) {
            if (blockIdx.x == 0 && threadIdx.x < kWave) {
                int *ls = reinterpret_cast<int *>(lds);
                plan_wave_body(wp.ids, wp.w, wp.nent, wp.E, wp.K, wp.tm, wp.nbits, wp.cnt,
                               wp.eoff, wp.boff, wp.tiles, wp.stok, wp.sw, wp.pos, wp.meta,
                               const_cast<int32_t *>(ctl), const_cast<WorkItem *>(items),
                               wp.max_items, wp.max_rows, 0, ls, ls + kMaxExperts);
            }
            return;  // (no barrier in these workgroups)
        }
        if (threadIdx.x < kWave) {
            int n, b;
            WorkItem w_it;
            wave_plan_item(wp.ids, wp.nent, wp.E, wp.K, wp.tm, wp.nbits, wp.max_rows, per_item,
                           blockIdx.x - 8, &n, &b, &w_it, s_tok);
            if (threadIdx.x == 0) {
                s_nb[0] = n;
                s_nb[1] = b;
                s_item = w_it;
            }
        }
        __syncthreads();
        const int nitems = s_nb[0], lb = s_nb[1];
        if (lb < 0) return;  // whole workgroup, after its only barrier outside the cell
        const WorkItem it = s_item;
        const int rem = lb - (lb / per_item) * per_item;
        const int g = rem / p.nsplit, split = rem - g * p.nsplit;
        const int kb = split * p.split_steps * KSTEP;
        const int ke = min(p.Kd, kb + p.split_steps * KSTEP);
        if (nitems * per_item < kDeepBelowCells)  // (no runs)
            single_cell<T, true, true, PACKED, true>(p, it, g, kb, ke, split, lds, rinfo, s_tok);
        else
            single_cell<T, true, true, PACKED, false>(p, it, g, kb, ke, split, lds, rinfo, s_tok);
    } else {
        const int nitems = ctl[0];
        const int ifirst = p.skip_quads ? min(ctl[1], nitems) : 0;
        const int lb = xcd_logical_block((nitems - ifirst) * per_item);
        if (lb < 0) return;  // whole workgroup: no barrier reached
        const int il = lb / per_item;  // item ifirst + il
        const int i = ifirst + il;
        const int rem = lb - il * per_item;
        const int g = rem / p.nsplit, split = rem - g * p.nsplit;
        const int kb = split * p.split_steps * KSTEP;
        const int ke = min(p.Kd, kb + p.split_steps * KSTEP);
        const WorkItem it = items[i];
        // weight-stream depth of the launch: deep when at least half the items
        // are in runs or when the cells do not fill the GPU's workgroup slots,
        // else shallow (the same for every workgroup)
        if (2 * ctl[2] >= nitems || (nitems - ifirst) * per_item < kDeepBelowCells)
            gemm_cell<T, GATEUP, GATHERED, PACKED, true>(p, items, it, i, nitems, g, kb, ke, split,
                                                         lds, rinfo);
        else
            gemm_cell<T, GATEUP, GATHERED, PACKED, false>(p, items, it, i, nitems, g, kb, ke,
                                                          split, lds, rinfo);
    }
}

// ---- big cells: runs of 4 items on 8 wavefronts (packed, 16-bit) ------------
// An expert with hundreds of rows (a long prompt in one call) turns its
// projections from weight streaming into dense GEMMs bound by the matrix
// cores; the 4-wavefront cells above then move too many operand bytes per
// MFMA. A big cell is one run of 4 items (up to 256 rows) x 256 weight
// columns (gate/up: 128 columns of h from each matrix; down: 256 columns of
// y) on 512 threads, in 32-wide K-steps:
//  * a step's operands (A: 256 rows x 64 bytes; B: the 4 KB packed tiles of
//    slices w0, w0+1, already in MFMA lane order) go straight from memory into
//    one of 5 LDS buffers of 32 KB (the whole LDS; buffer loads with the LDS
//    flag, no registers), 4 steps ahead of the MFMAs, and are waited for 2
//    steps before use: these loads spend about as long in the memory system as
//    a step's MFMAs take (the down epilogue's router weights are loaded into
//    registers at the start instead of LDS);
//  * the loads keep the default cache policy: the operands of a step are read
//    by several workgroups at about the same time (the rows by every column
//    block of the run, the weights by the runs of the same expert), which then
//    hit in L2 (non-temporal weight loads were measured 10% slower);
//  * the MFMA operands of step s+1 are read from LDS into registers while the
//    MFMAs of step s run, each into the register of the operand it replaces
//    once that operand's last MFMA is issued; one barrier per step, as inline
//    asm with a memory clobber (__syncthreads()'s release fence would wait for
//    every load in flight);
//  * in LDS the 16-byte chunk j of A row r sits at chunk j ^ ((r >> 1) & 3):
//    the MFMA-order reads are then free of bank conflicts;
//  * wavefront (wr, wc) computes rows 64*wr.. of the run and packed slice
//    w0 + wc: the same 2 x 4 x 4 accumulators, MFMA sequence and epilogue as
//    a tall cell, so the results are the same bits.
// The buffers are separate LDS arrays and the step loop is unrolled by 5, so
// that the compiler can tell a buffer's reads from the loads in flight into
// the others and does not make the reads wait for those loads.
constexpr int kBigThreads = 512;
constexpr int kDeepAU4 = 4 * kItemRows * 4;   // A tile of one step: 256 rows x 4 chunks
constexpr int kDeepBufU4 = kDeepAU4 + 1024;   // + B: 16 KB = 32 KB per buffer
template <typename T, bool GATEUP, bool GATHERED>
__global__ __launch_bounds__(kBigThreads) void k_big(const GemmArgs p,
                                                      const int32_t *__restrict__ ctl,
                                                      const WorkItem *__restrict__ items)
{
    static_assert(sizeof(T) == 2, "big cells: 16-bit element types");
    static_assert(GATEUP || !GATHERED, "the down projection reads h row-major");
    constexpr int ES = 2;
    constexpr int BCOLS = big_cols(GATEUP);
    constexpr int NB = 5;                     // LDS buffers
    constexpr int VM = 4 * (NB - 3);          // loads of this wavefront still in flight
    __shared__ uint4 L0[kDeepBufU4], L1[kDeepBufU4], L2[kDeepBufU4], L3[kDeepBufU4],
        L4[kDeepBufU4];
    const int Kd = p.Kd, N = p.N;
    const int ncb = (N + BCOLS - 1) / BCOLS;
    const int nquads = min(ctl[1], ctl[0]) / 4;
    const int lb = xcd_logical_block(nquads * ncb);
    if (lb < 0) return;  // whole workgroup: no barrier reached
    const int qd = lb / ncb, cb = lb - qd * ncb;
    const WorkItem first = items[4 * qd];
    const WorkItem last = items[4 * qd + 3];
    // workgroup-uniform by construction; said so, so that the buffer
    // descriptors built from them stay in scalar registers
    const int expert = __builtin_amdgcn_readfirstlane(first.expert);
    const int row0 = __builtin_amdgcn_readfirstlane(first.row0);
    const int nvalid = __builtin_amdgcn_readfirstlane(
        max(0, min(4 * kItemRows, last.row0 + last.nrows - row0)));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave & 3, wc = wave >> 2;
    const int nq = lane & 15, kg = lane >> 4;
    const WorkItem it = items[4 * qd + wr];
    // down: the router weight and token of the item's row 16 mt + 4 kg + r,
    // with (mt, r) = (nq >> 2, nq & 3), loaded now so that they have landed by
    // the epilogue; the 16 lanes of a K-group hold the 16 rows that each of
    // them stores (taken there with a shuffle), one register each
    float rsw = 0.f;
    int rtok = -1;
    if constexpr (!GATEUP) {
        const int rl = 16 * (nq >> 2) + 4 * kg + (nq & 3);
        if (rl < it.nrows) {
            rsw = p.sw[(int64_t)it.row0 + rl];
            rtok = p.stok[(int64_t)it.row0 + rl];
        }
    }

    // B: per step the packed tiles of slices w0, w0+1: gate/up 8 KB of gate,
    // then 8 KB of up; down 16 KB (tiles (w0, 0), (w0, 1), (w0+1, 0),
    // (w0+1, 1)). Wavefront w moves KB 2 w and 2 w + 1 of these 16.
    const PackedGeom z = packed_geom(Kd, N, GATEUP, ES);
    const int w0 = 2 * (cb & 1);
    const size_t gbase = ((size_t)expert * z.gs + (cb >> 1)) * z.nst * z.step_bytes;
    const uint32_t grange = (uint32_t)z.nst * z.step_bytes;
    __amdgpu_buffer_rsrc_t rb;
    uint32_t vb;
    if constexpr (GATEUP) {
        rb = make_rsrc(static_cast<const char *>(wave >> 2 ? p.B1 : p.B0) + gbase, grange);
        vb = (uint32_t)w0 * 4096u + (uint32_t)(wave & 3) * 2048u;
    } else {
        rb = make_rsrc(static_cast<const char *>(p.B0) + gbase, grange);
        vb = (uint32_t)w0 * 8192u + (uint32_t)wave * 2048u;
    }
    vb += (uint32_t)lane * 16u;
    const int bslot = kDeepAU4 + 128 * wave;

    // A: wavefront w moves rows 32 w .. 32 w + 31, 16 rows per instruction;
    // lane l takes row 32 w + 16 i + (l >> 2) and fills its LDS chunk l & 3
    // with the row's K chunk (l & 3) ^ ((l >> 3) & 3)
    const int arow = 32 * wave + (lane >> 2);
    const uint32_t achunk = (uint32_t)(8 * ((lane & 3) ^ ((lane >> 3) & 3)));  // elements
    __amdgpu_buffer_rsrc_t ra;
    uint32_t va[2];
    if constexpr (GATHERED) {
        ra = make_rsrc(p.A, (uint32_t)((size_t)p.a_rows * Kd * ES));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = arow + 16 * i;
            const int t = r < nvalid ? p.stok[row0 + r] : -1;
            va[i] = (unsigned)t < (unsigned)p.a_rows ? (uint32_t)t * (uint32_t)Kd * ES : 0x80000000u;
        }
    } else {
        ra = make_rsrc(static_cast<const T *>(p.A) + (size_t)row0 * Kd,
                       (uint32_t)((size_t)nvalid * Kd * ES));
#pragma unroll
        for (int i = 0; i < 2; ++i) va[i] = (uint32_t)(arow + 16 * i) * (uint32_t)Kd * ES;
    }

    float4_t acc[2][kMT][kNpl];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int c = 0; c < kNpl; ++c) acc[m][mt][c] = float4_t{0.f, 0.f, 0.f, 0.f};

    typedef __attribute__((address_space(3))) void *lds_ptr;
    // the operands of K-step s into LDS buffer L; K chunks past Kd (the next
    // row's data) and steps past the end are read at offsets past the
    // descriptors' ranges, which return zeros
    auto issue = [&](uint4 (&L)[kDeepBufU4], int s) {
        const uint32_t ka = (uint32_t)(32 * s) + achunk;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_ptr)(L + (32 * wave + 16 * i) * 4), 16,
                (int)ka < Kd ? va[i] + ka * ES : 0x80000000u, 0, 0, 0);
        const uint32_t o = vb + (uint32_t)s * z.step_bytes;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(L + bslot + 64 * j), 16,
                                                     o + (uint32_t)j * 1024u, 0, 0, 0);
    };
    uint4 fa[kMT], fb[2][kNpl];
    auto read_a = [&](const uint4 (&L)[kDeepBufU4]) {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
            const int row = 64 * wr + 16 * mt + nq;
            fa[mt] = L[row * 4 + (kg ^ ((row >> 1) & 3))];
        }
    };
    // B operand (matrix or slice half m, column quad c) of this wavefront
    auto read_b = [&](const uint4 (&L)[kDeepBufU4], int m, int c) {
        fb[m][c] = L[kDeepAU4 + (GATEUP ? 512 * m + 256 * wc : 512 * wc + 256 * m) + 64 * c + lane];
    };
    // step s: loads of step s+4 into Lf (read for step s-1, complete before
    // the last barrier), MFMAs of step s with step s+1's operands read from Ln
    // into the registers as they free up, then this wavefront's loads of step
    // s+2 landed, barrier
    auto stepfn = [&](int s, const uint4 (&Ln)[kDeepBufU4], uint4 (&Lf)[kDeepBufU4]) {
        issue(Lf, s + NB - 1);
#pragma unroll
        for (int c = 0; c < kNpl; ++c)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int mt = 0; mt < kMT; ++mt)
                    acc[m][mt][c] = Elt<T>::mfma(fa[mt], fb[m][c], acc[m][mt][c]);
                read_b(Ln, m, c);
                // keep this order: a read hoisted above the MFMAs would hold a
                // second set of operand registers
                __builtin_amdgcn_sched_barrier(0);
            }
        read_a(Ln);
        __builtin_amdgcn_s_waitcnt(wait_vm(VM));
        asm volatile("s_barrier" ::: "memory");
    };

    const int nst = z.nst;
    issue(L0, 0);
    issue(L1, 1);
    issue(L2, 2);
    issue(L3, 3);
    __builtin_amdgcn_s_waitcnt(wait_vm(VM));  // steps 0 and 1 landed
    asm volatile("s_barrier" ::: "memory");
    read_a(L0);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int c = 0; c < kNpl; ++c) read_b(L0, m, c);
    // (no early exits from the unrolled loop: they made the compiler spill)
    int s = 0;
    for (; s + 5 <= nst; s += 5) {
        stepfn(s, L1, L4);
        stepfn(s + 1, L2, L0);
        stepfn(s + 2, L3, L1);
        stepfn(s + 3, L4, L2);
        stepfn(s + 4, L0, L3);
    }
    if (s < nst) stepfn(s, L1, L4);
    if (s + 1 < nst) stepfn(s + 1, L2, L0);
    if (s + 2 < nst) stepfn(s + 2, L3, L1);
    if (s + 3 < nst) stepfn(s + 3, L4, L2);
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // no load into LDS in flight at exit
    const int col = BCOLS * cb + (BCOLS / 2) * wc + kNpl * nq;
    if constexpr (GATEUP) {
        store_cells<T, true, kMT, false>(p, it, col, kg, acc, nullptr, 0);
    } else {
        // y = router weight x accumulator (fp32) on rows holding an entry, as
        // store_cells does, through a descriptor over the item's rows (the
        // shuffles run with every lane of the wavefront active). Non-temporal
        // here: at the shapes that take big cells y is far larger than the
        // caches, and sc1 stores evicted the operands that the other
        // workgroups share in L2 (measured: down 1.83 -> 1.67 ms on the
        // one-call long prompt)
        constexpr int HALF = 16 * kNpl;
        if (p.yexp) {
            // compact y (binary16 + block exponents), the same rows and stores
            const int col0 = BCOLS * cb + (BCOLS / 2) * wc;
            if (col0 >= N) return;  // wave-uniform
            const __amdgpu_buffer_rsrc_t ry16 =
                make_rsrc(static_cast<uint16_t *>(p.out) + (int64_t)it.row0 * N,
                          (uint32_t)(it.nrows * N * 2));
            int ev[kMT][4];
#pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ev[mt][r] = 0;
                    const int src = 16 * kg + 4 * mt + r;
                    const float g = __shfl(rsw, src);
                    if (__shfl(rtok, src) < 0) continue;  // uniform over the DPP row
                    const int rl = 16 * mt + 4 * kg + r;
                    float v[2][4];
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int c = 0; c < 4; ++c) v[m][c] = g * acc[m][mt][c][r];
                    ev[mt][r] = store_y16_row(p, ry16, rl, col, v, 0);
                }
            // this lane holds the token of row 16 (nq >> 2) + 4 kg + (nq & 3)
            store_y16_exponents<kMT>(p.yexp + (col0 / kY16Block) * p.estride, it.row0, ev,
                                     16 * (nq >> 2) + 4 * kg + (nq & 3), rtok >= 0);
            return;
        }
        const __amdgpu_buffer_rsrc_t ry =
            make_rsrc(static_cast<float *>(p.out) + (int64_t)it.row0 * N, (uint32_t)(it.nrows * N * 4));
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int src = 16 * kg + 4 * mt + r;
                const float g = __shfl(rsw, src);
                if (__shfl(rtok, src) < 0) continue;  // pad rows (and rows past the item)
                const int rl = 16 * mt + 4 * kg + r;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    if (col + m * HALF >= N) continue;  // col + HALF < N implies col < N
                    const float4 v = make_float4(g * acc[m][mt][0][r], g * acc[m][mt][1][r],
                                                 g * acc[m][mt][2][r], g * acc[m][mt][3][r]);
                    store_sc1<kNT>(ry, (uint32_t)((rl * N + col + m * HALF) * 4), v);
                }
            }
    }
}

// ---- split-K reductions (fixed split order) --------------------------------
__device__ __forceinline__ int rows_of_plan(const int32_t *meta, int64_t max_rows)
{
    const int64_t nr = meta[kMetaNr];
    return (int)(nr < 0 ? 0 : (nr > max_rows ? max_rows : nr));
}

// Both reductions are instantiated per split count NS, so that the NS planes'
// loads are issued together rather than one loop trip at a time (a split
// layer is latency-bound); the sums stay in split order.

// h[r][c..c+3] = D(silu(sum_s G_s) * sum_s U_s) for rows r < nr; pad rows
// (stok < 0, whose partial sums are not stored) get h = 0, as unsplit
template <typename T, int NS>
__global__ __launch_bounds__(256) void k_reduce_gateup(const float *__restrict__ part,
                                                       int64_t plane, int N,
                                                       const int32_t *__restrict__ stok,
                                                       const int32_t *__restrict__ meta,
                                                       int64_t max_rows, T *__restrict__ h)
{
    const int per = N / 4;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = q / per;
    const int c = (int)(q - row * per) * 4;
    if (row >= rows_of_plan(meta, max_rows)) return;
    const float *P = part + row * 2 * N + c;
    float4 gs = make_float4(0.f, 0.f, 0.f, 0.f), us = gs;
    if (stok[row] >= 0) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float4 gv = *reinterpret_cast<const float4 *>(P + s * plane);
            const float4 uv = *reinterpret_cast<const float4 *>(P + s * plane + N);
            gs = make_float4(gs.x + gv.x, gs.y + gv.y, gs.z + gv.z, gs.w + gv.w);
            us = make_float4(us.x + uv.x, us.y + uv.y, us.z + uv.z, us.w + uv.w);
        }
    }
    const float h0 = silu(gs.x) * us.x, h1 = silu(gs.y) * us.y;
    const float h2 = silu(gs.z) * us.z, h3 = silu(gs.w) * us.w;
    T *H = h + row * N + c;
    if constexpr (sizeof(T) == 2)
        store_nt(reinterpret_cast<uint2 *>(H),
                 make_uint2(Elt<T>::pack2(h0, h1), Elt<T>::pack2(h2, h3)));
    else
        store_nt(reinterpret_cast<float4 *>(H), make_float4(h0, h1, h2, h3));
}

// y[r][c..c+3] = sw[r] * sum_s Y_s for rows r < nr with stok[r] >= 0
template <int NS>
__global__ __launch_bounds__(256) void k_reduce_down(const float *__restrict__ part, int64_t plane,
                                                     int N,
                                                     const int32_t *__restrict__ stok,
                                                     const float *__restrict__ sw,
                                                     const int32_t *__restrict__ meta,
                                                     int64_t max_rows, float *__restrict__ y)
{
    const int per = N / 4;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = q / per;
    const int c = (int)(q - row * per) * 4;
    if (row >= rows_of_plan(meta, max_rows) || stok[row] < 0) return;
    const float *P = part + row * N + c;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const float4 v = *reinterpret_cast<const float4 *>(P + s * plane);
        a = make_float4(a.x + v.x, a.y + v.y, a.z + v.z, a.w + v.w);
    }
    const float g = sw[row];
    store_nt(reinterpret_cast<float4 *>(y + row * N + c),
             make_float4(g * a.x, g * a.y, g * a.z, g * a.w));
}

// y in the compact format from the split planes: half a wavefront per (row,
// exponent block), lane l of it taking columns kY16Block * b + 4 l .. + 3; a
// unit's 32 lanes are all active or all not (the row decides), so the block
// maximum runs over all of them
template <int NS>
__global__ __launch_bounds__(256) void k_reduce_down_y16(
    const float *__restrict__ part, int64_t plane, int N, const int32_t *__restrict__ stok,
    const float *__restrict__ sw, const int32_t *__restrict__ meta, int64_t max_rows,
    uint16_t *__restrict__ y, int8_t *__restrict__ yexp, int nyb)
{
    // (exponents block-major: yexp[b * max_rows + row])
    const int64_t unit = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;
    const int l = threadIdx.x & 31;
    const int64_t row = unit / nyb;
    const int b = (int)(unit - row * nyb);
    if (row >= rows_of_plan(meta, max_rows) || stok[row] < 0) return;
    const int c = b * kY16Block + 4 * l;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < N) {
        const float *P = part + row * N + c;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float4 v = *reinterpret_cast<const float4 *>(P + s * plane);
            a = make_float4(a.x + v.x, a.y + v.y, a.z + v.z, a.w + v.w);
        }
    }
    const float g = sw[row];
    const float v[4] = {g * a.x, g * a.y, g * a.z, g * a.w};
    float M = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) M = __builtin_fmaxf(M, c < N ? __builtin_fabsf(v[q]) : 0.0f);
    M = row16_fmax(M);
    M = __builtin_fmaxf(M, __shfl_xor(M, 16));  // the unit's other 16 lanes
    const int e = y16_exponent(M);
    if (c < N) {
        const float scale = pow2f(e);
        float q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = v[k] * scale;
        store_nt(reinterpret_cast<uint2 *>(y + row * N + c),
                 make_uint2(Elt<_Float16>::pack2(q[0], q[1]), Elt<_Float16>::pack2(q[2], q[3])));
    }
    if (l == 0) yexp[b * max_rows + row] = (int8_t)e;
}

// ---- host launchers --------------------------------------------------------
// the reductions' launch for a split count in [2, kMaxSplit] (any other count
// is refused)
template <typename T, int NS = 2>
hipError_t reduce_gateup(int nsplit, dim3 grid, hipStream_t s, const float *part, int64_t plane, int N,
                   const int32_t *stok, const int32_t *meta, int64_t max_rows, T *h)
{
    if constexpr (NS <= kMaxSplit) {
        if (nsplit != NS)
            return reduce_gateup<T, NS + 1>(nsplit, grid, s, part, plane, N, stok, meta, max_rows,
                                            h);
        hipLaunchKernelGGL((k_reduce_gateup<T, NS>), grid, dim3(256), 0, s, part, plane, N, stok,
                           meta, max_rows, h);
        return hipSuccess;
    }
    return hipErrorInvalidValue;
}

template <int NS = 2>
hipError_t reduce_down(int nsplit, dim3 grid, hipStream_t s, const float *part, int64_t plane, int N,
                 const int32_t *stok, const float *sw, const int32_t *meta, int64_t max_rows,
                 float *y)
{
    if constexpr (NS <= kMaxSplit) {
        if (nsplit != NS)
            return reduce_down<NS + 1>(nsplit, grid, s, part, plane, N, stok, sw, meta, max_rows,
                                       y);
        hipLaunchKernelGGL((k_reduce_down<NS>), grid, dim3(256), 0, s, part, plane, N, stok, sw,
                           meta, max_rows, y);
        return hipSuccess;
    }
    return hipErrorInvalidValue;
}

template <int NS = 2>
hipError_t reduce_down_y16(int nsplit, dim3 grid, hipStream_t s, const float *part, int64_t plane,
                           int N, const int32_t *stok, const float *sw, const int32_t *meta,
                           int64_t max_rows, uint16_t *y, int8_t *yexp, int nyb)
{
    if constexpr (NS <= kMaxSplit) {
        if (nsplit != NS)
            return reduce_down_y16<NS + 1>(nsplit, grid, s, part, plane, N, stok, sw, meta,
                                           max_rows, y, yexp, nyb);
        hipLaunchKernelGGL((k_reduce_down_y16<NS>), grid, dim3(256), 0, s, part, plane, N, stok,
                           sw, meta, max_rows, y, yexp, nyb);
        return hipSuccess;
    }
    return hipErrorInvalidValue;
}

hipError_t launch_worklist(const int32_t *eoff, int E, int64_t max_rows, void *scratch,
                           int64_t max_items, bool runs_first, hipStream_t s)
{
    int32_t *ctl = static_cast<int32_t *>(scratch);
    WorkItem *items = reinterpret_cast<WorkItem *>(static_cast<char *>(scratch) + kCtlBytes);
    hipLaunchKernelGGL(k_worklist, dim3(1), dim3(1024), 0, s, eoff, E, max_rows, ctl, items,
                       (int)max_items, runs_first ? 1 : 0);
    return hipGetLastError();
}

namespace {

const int32_t *ctl_of(const void *scratch) { return static_cast<const int32_t *>(scratch); }
const WorkItem *items_of(const void *scratch)
{
    return reinterpret_cast<const WorkItem *>(static_cast<const char *>(scratch) + kCtlBytes);
}

GemmArgs gemm_args(const FfnShape &z, const void *scratch, bool gateup)
{
    GemmArgs p{};
    p.part = reinterpret_cast<float *>(static_cast<char *>(const_cast<void *>(scratch)) +
                                       z.part_offset);
    p.nsplit = gateup ? z.split_gu : z.split_dn;
    p.split_steps = gateup ? z.steps_gu : z.steps_dn;
    p.plane = gateup ? z.plane_gu : z.plane_dn;
    return p;
}

unsigned reduce_blocks(int64_t rows, int N) { return (unsigned)((rows * (N / 4) + 255) / 256); }

template <typename T, bool PACKED>
hipError_t gateup_t(const FfnShape &z, const void *a, int a_rows, bool gathered,
                    const int32_t *stok, const void *wg, const void *wu, int d, int f,
                    const int32_t *meta, const void *scratch, void *h, hipStream_t s,
                    const WavePlan *wp)
{
    GemmArgs p = gemm_args(z, scratch, true);
    p.A = a;
    p.a_rows = a_rows;
    p.B0 = wg;
    p.B1 = wu;
    p.stok = stok;
    p.out = h;
    p.Kd = d;
    p.N = f;
    const dim3 grid((unsigned)z.blocks_gu);
    if constexpr (PACKED && sizeof(T) == 2) {
        if (z.big_gu && z.blocks_big_gu > 0) {
            p.skip_quads = 1;
            const dim3 bgrid((unsigned)z.blocks_big_gu);
            if (gathered)
                hipLaunchKernelGGL((k_big<T, true, true>), bgrid, dim3(kBigThreads), 0, s, p,
                                   ctl_of(scratch), items_of(scratch));
            else
                hipLaunchKernelGGL((k_big<T, true, false>), bgrid, dim3(kBigThreads), 0, s, p,
                                   ctl_of(scratch), items_of(scratch));
        }
    }
    const WavePlan none{};
    if (gathered && wp && wp->ids)  // planned here: 8 workgroups before the cells'
        hipLaunchKernelGGL((k_expert_gemm<T, true, true, PACKED, true>), dim3(grid.x + 8),
                           dim3(256), 0, s, p, ctl_of(scratch), items_of(scratch), *wp);
    else if (gathered)  // rows gathered from x through stok
        hipLaunchKernelGGL((k_expert_gemm<T, true, true, PACKED>), grid, dim3(256), 0, s, p,
                           ctl_of(scratch), items_of(scratch), none);
    else
        hipLaunchKernelGGL((k_expert_gemm<T, true, false, PACKED>), grid, dim3(256), 0, s, p,
                           ctl_of(scratch), items_of(scratch), none);
    if (z.split_gu > 1) {
        const hipError_t e = reduce_gateup<T>(p.nsplit, dim3(reduce_blocks(z.max_rows, f)), s,
                                              p.part, p.plane, f, stok, meta, z.max_rows,
                                              static_cast<T *>(h));
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

template <typename T, bool PACKED>
hipError_t down_t(const FfnShape &z, const void *h, const void *wd, int d, int f,
                  const int32_t *stok, const float *sw, const int32_t *meta, const void *scratch,
                  void *y, int8_t *yexp, hipStream_t s)
{
    GemmArgs p = gemm_args(z, scratch, false);
    p.A = h;
    p.B0 = wd;
    p.stok = stok;
    p.sw = sw;
    p.out = y;
    p.Kd = f;
    p.N = d;
    int nyb = 0;
    if constexpr (sizeof(T) == 2) {
        p.yexp = yexp;
        p.estride = z.max_rows;
        nyb = (d + kY16Block - 1) / kY16Block;
    }
    if constexpr (PACKED && sizeof(T) == 2) {
        if (z.big_dn && z.blocks_big_dn > 0) {
            p.skip_quads = 1;
            hipLaunchKernelGGL((k_big<T, false, false>), dim3((unsigned)z.blocks_big_dn),
                               dim3(kBigThreads), 0, s, p, ctl_of(scratch), items_of(scratch));
        }
    }
    hipLaunchKernelGGL((k_expert_gemm<T, false, false, PACKED>), dim3((unsigned)z.blocks_dn),
                       dim3(256), 0, s, p, ctl_of(scratch), items_of(scratch), WavePlan{});
    if (z.split_dn > 1) {
        const hipError_t e =
            p.yexp ? reduce_down_y16(p.nsplit,
                                     dim3((unsigned)((z.max_rows * nyb * 32 + 255) / 256)), s,
                                     p.part, p.plane, d, stok, sw, meta, z.max_rows,
                                     static_cast<uint16_t *>(y), p.yexp, nyb)
                   : reduce_down(p.nsplit, dim3(reduce_blocks(z.max_rows, d)), s, p.part,
                                 p.plane, d, stok, sw, meta, z.max_rows, static_cast<float *>(y));
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t gateup_any(const FfnShape &z, bool packed, const void *a, int a_rows, bool gathered,
                      const int32_t *stok, const void *wg, const void *wu, int d, int f,
                      const int32_t *meta, const void *scratch, void *h, hipStream_t s,
                      const WavePlan *wp = nullptr)
{
    return packed ? gateup_t<T, true>(z, a, a_rows, gathered, stok, wg, wu, d, f, meta, scratch, h,
                                      s, wp)
                  : gateup_t<T, false>(z, a, a_rows, gathered, stok, wg, wu, d, f, meta, scratch, h,
                                       s, wp);
}

}  // namespace

hipError_t launch_gateup(const FfnShape &z, int dtype, bool packed, const void *xs,
                         const int32_t *stok, const void *wg, const void *wu, int d, int f,
                         const int32_t *meta, const void *scratch, void *h, hipStream_t s)
{
    if (dtype == 1)
        return gateup_any<_Float16>(z, packed, xs, 0, false, stok, wg, wu, d, f, meta, scratch, h, s);
    if (dtype == 2)
        return gateup_any<__bf16>(z, packed, xs, 0, false, stok, wg, wu, d, f, meta, scratch, h, s);
    return gateup_any<float>(z, packed, xs, 0, false, stok, wg, wu, d, f, meta, scratch, h, s);
}

hipError_t launch_gateup_gathered(const FfnShape &z, int dtype, bool packed, const void *x, int T,
                                  const int32_t *stok, const void *wg, const void *wu, int d, int f,
                                  const int32_t *meta, const void *scratch, void *h, hipStream_t s,
                                  const WavePlan *wp)
{
    if (dtype == 1)
        return gateup_any<_Float16>(z, packed, x, T, true, stok, wg, wu, d, f, meta, scratch, h, s,
                                    wp);
    if (dtype == 2)
        return gateup_any<__bf16>(z, packed, x, T, true, stok, wg, wu, d, f, meta, scratch, h, s,
                                  wp);
    return gateup_any<float>(z, packed, x, T, true, stok, wg, wu, d, f, meta, scratch, h, s, wp);
}

// every expert of a call of at most 64 entries pads to at most 64 rows (one
// work item) when tm divides 64
bool wave_plan_fits(int64_t nent, int tm) { return nent <= kWave && tm >= 1 && kWave % tm == 0; }

hipError_t launch_down(const FfnShape &z, int dtype, bool packed, const void *h, const void *wd,
                       int d, int f, const int32_t *stok, const float *sw, const int32_t *meta,
                       const void *scratch, void *y, int8_t *yexp, hipStream_t s)
{
    if (dtype == 1)
        return packed ? down_t<_Float16, true>(z, h, wd, d, f, stok, sw, meta, scratch, y, yexp, s)
                      : down_t<_Float16, false>(z, h, wd, d, f, stok, sw, meta, scratch, y, yexp, s);
    if (dtype == 2)
        return packed ? down_t<__bf16, true>(z, h, wd, d, f, stok, sw, meta, scratch, y, yexp, s)
                      : down_t<__bf16, false>(z, h, wd, d, f, stok, sw, meta, scratch, y, yexp, s);
    return packed ? down_t<float, true>(z, h, wd, d, f, stok, sw, meta, scratch, y, nullptr, s)
                  : down_t<float, false>(z, h, wd, d, f, stok, sw, meta, scratch, y, nullptr, s);
}

}  // namespace moe
