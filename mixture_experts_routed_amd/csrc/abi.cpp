// C ABI of the routed MoE layer (declared in include/moe_routed.h): argument
// checks on the host, then kernel launches on the caller's stream. No device
// allocation, no host synchronisation, no global mutable state.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <new>

#include "../../include/moe_routed.h"
#include "launch.hpp"

namespace {

constexpr int64_t kI32Max = 2147483647;

bool aligned(const void *p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : 2; }

bool dtype_ok(int dtype) { return dtype == MOE_F32 || dtype == MOE_F16 || dtype == MOE_BF16; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

hipStream_t as_stream(moe_stream_t s) { return static_cast<hipStream_t>(s); }

int plan_sizes(int T, int K, int E, int tm, moe_plan_sizes_t *o)
{
    if (T < 1 || K < 1 || E < 1 || tm < 1) return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
    const int64_t nent = (int64_t)T * K;
    if (nent > kI32Max - MOE_PLAN_BLOCK) return MOE_EINVAL;
    const int64_t act = nent < E ? nent : E;
    const int64_t rows = (nent + act * (tm - 1) + tm - 1) / tm * tm;
    if (rows > kI32Max - 1024) return MOE_EINVAL;
    o->nent = nent;
    o->nblk = (nent + MOE_PLAN_BLOCK - 1) / MOE_PLAN_BLOCK;
    o->max_rows = rows;
    o->max_tiles = rows / tm;
    o->scratch_bytes = (size_t)o->nblk * (size_t)(E + 2) * sizeof(int32_t);
    return MOE_OK;
}

int ffn_check(const void *xs, const void *wg, const void *wu, const void *wd, int dtype, int E,
              int d, int f, int tm, const int32_t *eoff, const int32_t *stok, const float *sw,
              const int32_t *meta, int64_t max_rows, const void *h, const float *y,
              const void *scratch, size_t scratch_bytes)
{
    if (!dtype_ok(dtype) || E < 1 || tm < 1 || d < 8 || f < 8 || d % 8 || f % 8 || max_rows < 1 ||
        max_rows > kI32Max - 1024)
        return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
    if (max_rows * (int64_t)(d > f ? d : f) > ((int64_t)1 << 40)) return MOE_EINVAL;
    // one expert matrix, and a work item's 64 rows of h or y, are each addressed
    // by one buffer descriptor (32-bit offsets)
    if ((int64_t)d * f * elem_bytes(dtype) > ((int64_t)1 << 31)) return MOE_EINVAL;
    if (d > (1 << 22) || f > (1 << 22)) return MOE_EINVAL;
    if (!aligned(xs, 16) || !aligned(wg, 16) || !aligned(wu, 16) || !aligned(wd, 16) ||
        !aligned(h, 16) || !aligned(y, 16) || !aligned(eoff, 4) || !aligned(stok, 4) ||
        !aligned(sw, 4) || !aligned(meta, 4) || !aligned(scratch, 16))
        return MOE_EINVAL;
    const moe::FfnShape z = moe::ffn_shape(E, tm, max_rows, d, f, dtype);
    if (z.blocks_gu > kI32Max || z.blocks_dn > kI32Max || z.blocks_big_gu > kI32Max ||
        z.blocks_big_dn > kI32Max)
        return MOE_EINVAL;
    if (scratch_bytes < z.scratch_bytes) return MOE_EINVAL;
    return MOE_OK;
}

// Record an event pair around each kernel when a timer is attached.
}  // namespace

struct moe_timer {
    int capacity;
    unsigned mask;
    int used[MOE_STAGE_N];
    hipEvent_t *ev[MOE_STAGE_N];  // 2 * capacity events per stage
};

namespace {

struct Rec {
    moe_timer_t *t;
    hipStream_t s;
    int stage;
    bool on;
    Rec(moe_timer_t *t_, hipStream_t s_, int stage_) : t(t_), s(s_), stage(stage_), on(false)
    {
        if (t && ((t->mask >> stage) & 1u) && t->used[stage] < t->capacity) {
            (void)hipEventRecord(t->ev[stage][2 * t->used[stage]], s);
            on = true;
        }
    }
    ~Rec()
    {
        if (on) {
            (void)hipEventRecord(t->ev[stage][2 * t->used[stage] + 1], s);
            t->used[stage]++;
        }
    }
};

// the work list puts the runs of 4 first when a big-cell kernel takes them
// (packed weights, 16-bit, shape as ffn_shape decides)
bool runs_first(const moe::FfnShape &z, bool packed) { return packed && (z.big_gu || z.big_dn); }

bool timer_room(const moe_timer_t *t)
{
    if (!t) return true;
    for (int q = 0; q < MOE_STAGE_N; ++q)
        if (((t->mask >> q) & 1u) && t->used[q] >= t->capacity) return false;
    return true;
}

// ffn_scratch != nullptr (moe_forward only): the plan also writes the grouped
// FFN's work list when it runs as one fused launch; *items_done says so.
int plan_impl(const int32_t *ids, const float *w, int T, int K, int E, int tm, int32_t *cnt,
              int32_t *eoff, int32_t *tiles, int32_t *stok, float *sw, int32_t *pos, int32_t *boff,
              int32_t *meta, void *scratch, size_t scratch_bytes, hipStream_t s, moe_timer_t *tmr,
              void *ffn_scratch = nullptr, bool *items_done = nullptr, bool runs_first = false)
{
    moe_plan_sizes_t z;
    const int rc = plan_sizes(T, K, E, tm, &z);
    if (rc != MOE_OK) return rc;
    if (!aligned(ids, 4) || !aligned(w, 4) || !aligned(cnt, 4) || !aligned(eoff, 4) ||
        !aligned(tiles, 4) || !aligned(stok, 4) || !aligned(sw, 4) || !aligned(pos, 4) ||
        !aligned(boff, 4) || !aligned(meta, 4) || !aligned(scratch, 4) ||
        scratch_bytes < z.scratch_bytes)
        return MOE_EINVAL;
    const int nent = (int)z.nent, nblk = (int)z.nblk;
    if (items_done) *items_done = false;
    if (nblk <= moe::plan_fused_max_blocks()) {
        // one launch: histogram, scan, pad fill and placement (timed as the placement)
        Rec r(tmr, s, MOE_STAGE_PLACE);
        const int64_t max_items = moe::ffn_max_items(E, tm, z.max_rows);
        if (moe::launch_plan_fused(ids, w, nent, E, K, tm, nblk, cnt, eoff, boff, tiles, stok, sw,
                                   pos, meta, ffn_scratch, max_items, z.max_rows, runs_first,
                                   s) != hipSuccess)
            return MOE_EHIP;
        if (items_done) *items_done = ffn_scratch != nullptr;
        return MOE_OK;
    }
    int32_t *bcnt = static_cast<int32_t *>(scratch);
    {
        Rec r(tmr, s, MOE_STAGE_HIST);
        if (moe::launch_hist(ids, nent, E, nblk, bcnt, s) != hipSuccess) return MOE_EHIP;
    }
    {
        Rec r(tmr, s, MOE_STAGE_SCAN);
        if (moe::launch_scan(bcnt, nblk, E, K, tm, nent, cnt, eoff, boff, tiles, stok, sw, meta,
                             s) != hipSuccess)
            return MOE_EHIP;
    }
    {
        Rec r(tmr, s, MOE_STAGE_PLACE);
        if (moe::launch_place(ids, w, nent, E, K, nblk, eoff, boff, stok, sw, pos, s) != hipSuccess)
            return MOE_EHIP;
    }
    return MOE_OK;
}

int gather_impl(const void *x, int dtype, int T, int d, const int32_t *stok, const int32_t *meta,
                int64_t max_rows, void *xs, hipStream_t s, moe_timer_t *tmr)
{
    if (!dtype_ok(dtype) || T < 1 || d < 8 || d % 8 || max_rows < 1 || max_rows > kI32Max)
        return MOE_EINVAL;
    if (!aligned(x, 16) || !aligned(xs, 16) || !aligned(stok, 4) || !aligned(meta, 4))
        return MOE_EINVAL;
    Rec r(tmr, s, MOE_STAGE_GATHER);
    if (moe::launch_gather(x, elem_bytes(dtype), T, d, stok, meta, max_rows, xs, s) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

// x != nullptr (moe_forward only): the gate/up kernel reads its rows from
// x[stok[r]] (T rows) and xs is not used.
// yexp != nullptr (moe_forward with 16-bit types): y receives the compact
// format (binary16 rows, then yexp's block exponents) instead of fp32 rows.
int ffn_impl(const void *xs, const void *wg, const void *wu, const void *wd, int dtype, int E,
             int d, int f, int tm, const int32_t *eoff, const int32_t *stok, const float *sw,
             const int32_t *meta, int64_t max_rows, void *h, float *y, void *scratch,
             size_t scratch_bytes, hipStream_t s, moe_timer_t *tmr, bool have_items = false,
             const void *x = nullptr, int T = 0, bool packed = false, int8_t *yexp = nullptr,
             const moe::WavePlan *wp = nullptr)
{
    const int rc = ffn_check(xs, wg, wu, wd, dtype, E, d, f, tm, eoff, stok, sw, meta, max_rows, h,
                             y, scratch, scratch_bytes);
    if (rc != MOE_OK) return rc;
    const moe::FfnShape z = moe::ffn_shape(E, tm, max_rows, d, f, dtype);
    if (!have_items) {
        Rec r(tmr, s, MOE_STAGE_WORKLIST);
        if (moe::launch_worklist(eoff, E, max_rows, scratch, z.max_items, runs_first(z, packed),
                                 s) != hipSuccess)
            return MOE_EHIP;
    }
    {
        Rec r(tmr, s, MOE_STAGE_GATEUP);
        const hipError_t e =
            x ? moe::launch_gateup_gathered(z, dtype, packed, x, T, stok, wg, wu, d, f, meta,
                                            scratch, h, s, wp)
              : moe::launch_gateup(z, dtype, packed, xs, stok, wg, wu, d, f, meta, scratch, h, s);
        if (e != hipSuccess) return MOE_EHIP;
    }
    {
        Rec r(tmr, s, MOE_STAGE_DOWN);
        if (moe::launch_down(z, dtype, packed, h, wd, d, f, stok, sw, meta, scratch, y, yexp, s) !=
            hipSuccess)
            return MOE_EHIP;
    }
    return MOE_OK;
}

// yexp != nullptr: y holds the compact format (see ffn_impl)
int combine_impl(const float *y, int64_t max_rows, const int32_t *pos, int T, int K, int d,
                 float *out, hipStream_t s, moe_timer_t *tmr, const int8_t *yexp = nullptr)
{
    if (T < 1 || K < 1 || d < 8 || d % 8 || max_rows < 1 || (int64_t)T * K > kI32Max)
        return MOE_EINVAL;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(pos, 4)) return MOE_EINVAL;
    Rec r(tmr, s, MOE_STAGE_COMBINE);
    const hipError_t e =
        yexp ? moe::launch_combine_y16(reinterpret_cast<const uint16_t *>(y), yexp, max_rows, pos,
                                       T, K, d, out, s)
             : moe::launch_combine(y, max_rows, pos, T, K, d, out, s);
    return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

int layout_impl(int T, int K, int E, int d, int f, int tm, int dtype, moe_forward_layout_t *L,
                moe_plan_sizes_t *z)
{
    if (!L || !dtype_ok(dtype) || d < 8 || f < 8 || d % 8 || f % 8) return MOE_EINVAL;
    const int rc = plan_sizes(T, K, E, tm, z);
    if (rc != MOE_OK) return rc;
    const size_t A = 256, es = (size_t)elem_bytes(dtype), R = (size_t)z->max_rows;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = round_up(o + bytes, A);
        return at;
    };
    L->cnt = take((size_t)E * 4);
    L->eoff = take((size_t)(E + 1) * 4);
    L->tiles = take((size_t)z->max_tiles * 4);
    L->stok = take(R * 4);
    L->sw = take(R * 4);
    L->pos = take((size_t)z->nent * 4);
    L->boff = take((size_t)z->nblk * E * 4);
    L->meta = take(MOE_META_N * 4);
    L->plan_scratch = take(z->scratch_bytes);
    L->xs = take(R * d * es);
    L->h = take(R * f * es);
    L->y = take(R * d * 4);
    L->ffn_scratch = take(moe::ffn_shape(E, tm, z->max_rows, d, f, dtype).scratch_bytes);
    L->total = o;
    return MOE_OK;
}

// Expert weights in host memory: the device cache's layout for S slots (the
// state: a 256-byte header with the ring hand and the last call's copy count,
// slot_of[E], exp_of[S], copy[S]; then S slots of each matrix at the layout's
// per-expert stride).
struct HostCache {
    int E, S;
    size_t bgu, bdn;  // bytes per slot: gate (= up), down
    size_t hdr, slot_of, exp_of, copy, gate, up, down, total;
};

int host_cache_layout(int E, int d, int f, int dtype, int packed, int S, HostCache *c)
{
    if (E < 1 || !dtype_ok(dtype) || d < 8 || f < 8 || d % 8 || f % 8 ||
        (packed != 0 && packed != 1))
        return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
    if (S < 1 || S > E) return MOE_EINVAL;
    const size_t es = elem_bytes(dtype);
    c->E = E;
    c->S = S;
    c->bgu = packed ? moe::packed_weight_bytes(1, d, f, true, dtype) : (size_t)d * f * es;
    c->bdn = packed ? moe::packed_weight_bytes(1, f, d, false, dtype) : (size_t)f * d * es;
    auto r256 = [](size_t v) { return (v + 255) / 256 * 256; };
    c->hdr = 0;
    c->slot_of = 256;
    c->exp_of = r256(c->slot_of + (size_t)E * 4);
    c->copy = r256(c->exp_of + (size_t)S * 4);
    c->gate = r256(c->copy + (size_t)S * 4);
    c->up = r256(c->gate + (size_t)S * c->bgu);
    c->down = r256(c->up + (size_t)S * c->bgu);
    c->total = r256(c->down + (size_t)S * c->bdn);
    return MOE_OK;
}

// the fewest slots that hold every expert one call of T tokens, top-K, routes to
int64_t host_cache_min_slots(int T, int K, int E)
{
    return (int64_t)T * K < E ? (int64_t)T * K : E;
}

moe::CacheState cache_state(const HostCache &c, void *cache)
{
    char *b = static_cast<char *>(cache);
    moe::CacheState st;
    st.hdr = reinterpret_cast<int32_t *>(b + c.hdr);
    st.slot_of = reinterpret_cast<int32_t *>(b + c.slot_of);
    st.exp_of = reinterpret_cast<int32_t *>(b + c.exp_of);
    st.copy = reinterpret_cast<int32_t *>(b + c.copy);
    st.gate = b + c.gate;
    st.up = b + c.up;
    st.down = b + c.down;
    st.bytes_gu = c.bgu;
    st.bytes_dn = c.bdn;
    st.E = c.E;
    st.S = c.S;
    return st;
}

// The device address of pinned, device-mapped host memory at p, or nullptr for
// anything else (pageable host memory, device memory), which the staging
// kernel must not be given. A failed query's error is cleared here.
const void *mapped_host(const void *p)
{
    if (!p) return nullptr;
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (a.type != hipMemoryTypeHost || !a.devicePointer || !a.hostPointer) return nullptr;
    return static_cast<const char *>(a.devicePointer) +
           (static_cast<const char *>(p) - static_cast<const char *>(a.hostPointer));
}

// Staging of host-resident weights inside a forward call
struct HostStage {
    const void *hg, *hu, *hd;  // device addresses of the host weights
    moe::CacheState st;
    int64_t max_new;
};

int forward_impl(const void *x, const int32_t *ids, const float *w, const void *wg, const void *wu,
                 const void *wd, int dtype, int T, int K, int E, int d, int f, int tm, void *ws,
                 size_t ws_bytes, float *out, hipStream_t s, moe_timer_t *tmr, bool packed = false,
                 const HostStage *hs = nullptr)
{
    moe_forward_layout_t L;
    moe_plan_sizes_t z;
    int rc = layout_impl(T, K, E, d, f, tm, dtype, &L, &z);
    if (rc != MOE_OK) return rc;
    if (!aligned(ws, 256) || ws_bytes < L.total || !aligned(x, 16) || !aligned(out, 16) ||
        !aligned(wg, 16) || !aligned(wu, 16) || !aligned(wd, 16))
        return MOE_EINVAL;
    if (!timer_room(tmr)) return MOE_EINVAL;
    char *b = static_cast<char *>(ws);
    auto i32 = [&](size_t off) { return reinterpret_cast<int32_t *>(b + off); };
    auto f32 = [&](size_t off) { return reinterpret_cast<float *>(b + off); };
    bool items = false;
    const moe::FfnShape fz = moe::ffn_shape(E, tm, z.max_rows, d, f, dtype);
    // The gate/up kernel gathers its rows from x itself when x is addressable
    // by one buffer descriptor (< 2 GiB); otherwise the rows are gathered first.
    const bool fused_gather = (size_t)T * d * elem_bytes(dtype) < ((size_t)1 << 31);
    // A call of at most one wavefront of entries, one work item per expert, is
    // planned inside the gate/up launch (moe::WavePlan): one launch fewer. Not
    // with host weights (the cache is assigned between the plan and the
    // GEMMs) nor with big cells (their launch precedes gate/up's).
    moe::WavePlan wp{};
    if (!hs && fused_gather && moe::wave_plan_fits((int64_t)T * K, tm) && !fz.big_gu &&
        !fz.big_dn) {
        if (!aligned(ids, 4) || !aligned(w, 4)) return MOE_EINVAL;
        int nbits = 0;
        while ((1 << nbits) < E) ++nbits;
        wp = moe::WavePlan{ids, w, T * K, E, K, tm, nbits, (int)fz.max_items, (int)z.max_rows,
                           i32(L.cnt), i32(L.eoff), i32(L.boff), i32(L.tiles), i32(L.stok),
                           f32(L.sw), i32(L.pos), i32(L.meta)};
        items = true;
    } else {
        rc = plan_impl(ids, w, T, K, E, tm, i32(L.cnt), i32(L.eoff), i32(L.tiles), i32(L.stok),
                       f32(L.sw), i32(L.pos), i32(L.boff), i32(L.meta), b + L.plan_scratch,
                       z.scratch_bytes, s, tmr, b + L.ffn_scratch, &items, runs_first(fz, packed));
        if (rc != MOE_OK) return rc;
    }
    if (hs) {
        // the routed experts' weights into the cache, the work list to slots
        if (!items) {
            if (moe::launch_worklist(i32(L.eoff), E, z.max_rows, b + L.ffn_scratch, fz.max_items,
                                     runs_first(fz, packed), s) != hipSuccess)
                return MOE_EHIP;
            items = true;
        }
        if (moe::launch_cache_stage(hs->st, i32(L.cnt), b + L.ffn_scratch, hs->hg, hs->hu, hs->hd,
                                    hs->max_new, s) != hipSuccess)
            return MOE_EHIP;
        wg = hs->st.gate;
        wu = hs->st.up;
        wd = hs->st.down;
    }
    if (!fused_gather) {
        rc = gather_impl(x, dtype, T, d, i32(L.stok), i32(L.meta), z.max_rows, b + L.xs, s, tmr);
        if (rc != MOE_OK) return rc;
    }
    // 16-bit types: the expert outputs in the compact format, binary16 rows at
    // L.y and their block exponents right after them (2d + ceil(d/128) bytes per
    // row fit in the region's 4d)
    int8_t *yexp = dtype == MOE_F32
                       ? nullptr
                       : reinterpret_cast<int8_t *>(b + L.y + (size_t)z.max_rows * d * 2);
    rc = ffn_impl(b + L.xs, wg, wu, wd, dtype, E, d, f, tm, i32(L.eoff), i32(L.stok), f32(L.sw),
                  i32(L.meta), z.max_rows, b + L.h, f32(L.y), b + L.ffn_scratch,
                  fz.scratch_bytes, s, tmr, items,
                  fused_gather ? x : nullptr, T, packed, yexp, wp.ids ? &wp : nullptr);
    if (rc != MOE_OK) return rc;
    return combine_impl(f32(L.y), z.max_rows, i32(L.pos), T, K, d, out, s, tmr, yexp);
}

}  // namespace

extern "C" {

int moe_route_topk(const float *logits, int T, int E, int K, int32_t *ids, float *w,
                   moe_stream_t stream)
{
    if (T < 1 || E < 1 || K < 1 || K > E) return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS || K > MOE_ROUTE_MAX_K) return MOE_EUNSUPPORTED;
    if ((int64_t)T * E > kI32Max * 4 || (int64_t)T * K > kI32Max) return MOE_EINVAL;
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(w, 4)) return MOE_EINVAL;
    if (moe::launch_route_topk(logits, T, E, K, ids, w, as_stream(stream)) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

int moe_plan_sizes(int T, int K, int E, int tm, moe_plan_sizes_t *out)
{
    if (!out) return MOE_EINVAL;
    return plan_sizes(T, K, E, tm, out);
}

int moe_plan(const int32_t *ids, const float *w, int T, int K, int E, int tm, int32_t *cnt,
             int32_t *eoff, int32_t *tiles, int32_t *stok, float *sw, int32_t *pos, int32_t *boff,
             int32_t *meta, void *scratch, size_t scratch_bytes, moe_stream_t stream)
{
    return plan_impl(ids, w, T, K, E, tm, cnt, eoff, tiles, stok, sw, pos, boff, meta, scratch,
                     scratch_bytes, as_stream(stream), nullptr);
}

int moe_gather(const void *x, int dtype, int T, int d, const int32_t *stok, const int32_t *meta,
               int64_t max_rows, void *xs, moe_stream_t stream)
{
    return gather_impl(x, dtype, T, d, stok, meta, max_rows, xs, as_stream(stream), nullptr);
}

int moe_ffn_scratch_bytes(int E, int d, int f, int tm, int64_t max_rows, int dtype,
                          size_t *bytes)
{
    if (!bytes || E < 1 || tm < 1 || max_rows < 1 || max_rows > kI32Max - 1024 ||
        !dtype_ok(dtype) || d < 8 || f < 8 || d % 8 || f % 8)
        return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
    *bytes = moe::ffn_shape(E, tm, max_rows, d, f, dtype).scratch_bytes;
    return MOE_OK;
}

int moe_ffn_splits(int E, int d, int f, int tm, int64_t max_rows, int dtype, int *split_gateup,
                   int *split_down)
{
    if (!split_gateup || !split_down || E < 1 || tm < 1 || max_rows < 1 ||
        max_rows > kI32Max - 1024 || !dtype_ok(dtype) || d < 8 || f < 8 || d % 8 || f % 8)
        return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
    const moe::FfnShape z = moe::ffn_shape(E, tm, max_rows, d, f, dtype);
    *split_gateup = z.split_gu;
    *split_down = z.split_dn;
    return MOE_OK;
}

int moe_ffn_big_cells(int E, int d, int f, int tm, int64_t max_rows, int dtype, int *on)
{
    if (!on || E < 1 || tm < 1 || max_rows < 1 || max_rows > kI32Max - 1024 || !dtype_ok(dtype) ||
        d < 8 || f < 8 || d % 8 || f % 8)
        return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
    const moe::FfnShape z = moe::ffn_shape(E, tm, max_rows, d, f, dtype);
    *on = (z.big_gu ? 1 : 0) | (z.big_dn ? 2 : 0);
    return MOE_OK;
}

int moe_expert_ffn(const void *xs, const void *w_gate, const void *w_up, const void *w_down,
                   int dtype, int E, int d, int f, int tm, const int32_t *eoff, const int32_t *stok,
                   const float *sw, const int32_t *meta, int64_t max_rows, void *h, float *y,
                   void *scratch, size_t scratch_bytes, moe_stream_t stream)
{
    return ffn_impl(xs, w_gate, w_up, w_down, dtype, E, d, f, tm, eoff, stok, sw, meta, max_rows, h,
                    y, scratch, scratch_bytes, as_stream(stream), nullptr);
}

int moe_packed_weight_bytes(int E, int d, int f, int dtype, int kind, size_t *bytes)
{
    if (!bytes || E < 1 || !dtype_ok(dtype) || d < 8 || f < 8 || d % 8 || f % 8 ||
        (kind != MOE_W_GATE_UP && kind != MOE_W_DOWN))
        return MOE_EINVAL;
    if (E > MOE_MAX_EXPERTS) return MOE_EUNSUPPORTED;
    const bool gu = kind == MOE_W_GATE_UP;
    *bytes = moe::packed_weight_bytes(E, gu ? d : f, gu ? f : d, gu, dtype);
    return MOE_OK;
}

int moe_pack_weights(const void *w, int dtype, int E, int d, int f, int kind, void *packed,
                     size_t packed_bytes, moe_stream_t stream)
{
    size_t need = 0;
    const int rc = moe_packed_weight_bytes(E, d, f, dtype, kind, &need);
    if (rc != MOE_OK) return rc;
    if (!aligned(w, 16) || !aligned(packed, 16) || packed_bytes < need) return MOE_EINVAL;
    if ((int64_t)d * f * elem_bytes(dtype) > ((int64_t)1 << 31)) return MOE_EINVAL;
    const bool gu = kind == MOE_W_GATE_UP;
    if (moe::launch_pack(dtype, w, E, gu ? d : f, gu ? f : d, gu, packed, as_stream(stream)) !=
        hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

int moe_expert_ffn_packed(const void *xs, const void *pw_gate, const void *pw_up,
                          const void *pw_down, int dtype, int E, int d, int f, int tm,
                          const int32_t *eoff, const int32_t *stok, const float *sw,
                          const int32_t *meta, int64_t max_rows, void *h, float *y, void *scratch,
                          size_t scratch_bytes, moe_stream_t stream)
{
    return ffn_impl(xs, pw_gate, pw_up, pw_down, dtype, E, d, f, tm, eoff, stok, sw, meta,
                    max_rows, h, y, scratch, scratch_bytes, as_stream(stream), nullptr, false,
                    nullptr, 0, true);
}

int moe_forward_packed(const void *x, const int32_t *ids, const float *w, const void *pw_gate,
                       const void *pw_up, const void *pw_down, int dtype, int T, int K, int E,
                       int d, int f, int tm, void *workspace, size_t ws_bytes, float *out,
                       moe_stream_t stream)
{
    return forward_impl(x, ids, w, pw_gate, pw_up, pw_down, dtype, T, K, E, d, f, tm, workspace,
                        ws_bytes, out, as_stream(stream), nullptr, true);
}

int moe_forward_packed_timed(const void *x, const int32_t *ids, const float *w,
                             const void *pw_gate, const void *pw_up, const void *pw_down,
                             int dtype, int T, int K, int E, int d, int f, int tm,
                             void *workspace, size_t ws_bytes, float *out, moe_stream_t stream,
                             moe_timer_t *timer)
{
    return forward_impl(x, ids, w, pw_gate, pw_up, pw_down, dtype, T, K, E, d, f, tm, workspace,
                        ws_bytes, out, as_stream(stream), timer, true);
}

int moe_host_cache_bytes(int T, int K, int E, int d, int f, int dtype, int packed, int slots,
                         size_t *bytes)
{
    if (!bytes || T < 1 || K < 1 || K > E || (int64_t)T * K > kI32Max || slots < 0) return MOE_EINVAL;
    const int64_t smin = host_cache_min_slots(T, K, E);
    if (slots != 0 && slots < smin) return MOE_EINVAL;
    HostCache c;
    const int rc = host_cache_layout(E, d, f, dtype, packed, slots ? slots : (int)smin, &c);
    if (rc == MOE_OK) *bytes = c.total;
    return rc;
}

int moe_host_cache_init(void *cache, size_t cache_bytes, int E, int d, int f, int dtype,
                        int packed, int slots, moe_stream_t stream)
{
    HostCache c;
    const int rc = host_cache_layout(E, d, f, dtype, packed, slots, &c);
    if (rc != MOE_OK) return rc;
    if (!cache || !aligned(cache, 256) || cache_bytes < c.total) return MOE_EINVAL;
    if (moe::launch_cache_clear(cache_state(c, cache), as_stream(stream)) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

int moe_forward_host_weights(const void *x, const int32_t *ids, const float *w,
                             const void *w_gate_host, const void *w_up_host,
                             const void *w_down_host, int packed, int dtype, int T, int K, int E,
                             int d, int f, int tm, int slots, void *cache, size_t cache_bytes,
                             void *workspace, size_t ws_bytes, float *out, moe_stream_t stream)
{
    if (T < 1 || K < 1 || K > E || (int64_t)T * K > kI32Max) return MOE_EINVAL;
    HostCache c;
    int rc = host_cache_layout(E, d, f, dtype, packed, slots, &c);
    if (rc != MOE_OK) return rc;
    const int64_t smin = host_cache_min_slots(T, K, E);
    if (slots < smin || !cache || !aligned(cache, 256) || cache_bytes < c.total ||
        !w_gate_host || !w_up_host || !w_down_host || !x || !ids || !w || !workspace || !out)
        return MOE_EINVAL;
    HostStage hs;
    hs.hg = mapped_host(w_gate_host);
    hs.hu = mapped_host(w_up_host);
    hs.hd = mapped_host(w_down_host);
    if (!hs.hg || !hs.hu || !hs.hd || !aligned(hs.hg, 16) || !aligned(hs.hu, 16) ||
        !aligned(hs.hd, 16))
        return MOE_EINVAL;
    hs.st = cache_state(c, cache);
    hs.max_new = smin;
    // the cache's matrices stand in for the device weights (checked as such)
    return forward_impl(x, ids, w, hs.st.gate, hs.st.up, hs.st.down, dtype, T, K, E, d, f, tm,
                        workspace, ws_bytes, out, as_stream(stream), nullptr, packed != 0, &hs);
}

int moe_combine(const float *y, int64_t max_rows, const int32_t *pos, int T, int K, int d,
                float *out, moe_stream_t stream)
{
    return combine_impl(y, max_rows, pos, T, K, d, out, as_stream(stream), nullptr);
}

int moe_forward_layout(int T, int K, int E, int d, int f, int tm, int dtype,
                       moe_forward_layout_t *out)
{
    moe_plan_sizes_t z;
    return layout_impl(T, K, E, d, f, tm, dtype, out, &z);
}

int moe_forward_workspace(int T, int K, int E, int d, int f, int tm, int dtype, size_t *bytes)
{
    if (!bytes) return MOE_EINVAL;
    moe_forward_layout_t L;
    moe_plan_sizes_t z;
    const int rc = layout_impl(T, K, E, d, f, tm, dtype, &L, &z);
    if (rc == MOE_OK) *bytes = L.total;
    return rc;
}

int moe_forward(const void *x, const int32_t *ids, const float *w, const void *w_gate,
                const void *w_up, const void *w_down, int dtype, int T, int K, int E, int d, int f,
                int tm, void *workspace, size_t ws_bytes, float *out, moe_stream_t stream)
{
    return forward_impl(x, ids, w, w_gate, w_up, w_down, dtype, T, K, E, d, f, tm, workspace,
                        ws_bytes, out, as_stream(stream), nullptr);
}

int moe_forward_timed(const void *x, const int32_t *ids, const float *w, const void *w_gate,
                      const void *w_up, const void *w_down, int dtype, int T, int K, int E, int d,
                      int f, int tm, void *workspace, size_t ws_bytes, float *out,
                      moe_stream_t stream, moe_timer_t *timer)
{
    return forward_impl(x, ids, w, w_gate, w_up, w_down, dtype, T, K, E, d, f, tm, workspace,
                        ws_bytes, out, as_stream(stream), timer);
}

int moe_timer_create(moe_timer_t **out, int capacity, unsigned stage_mask)
{
    if (!out || capacity < 1 || capacity > (1 << 20)) return MOE_EINVAL;
    if (stage_mask == 0 || (stage_mask >> MOE_STAGE_N) != 0) return MOE_EINVAL;
    moe_timer_t *t = new (std::nothrow) moe_timer_t();
    if (!t) return MOE_EINVAL;
    t->capacity = capacity;
    t->mask = stage_mask;
    for (int q = 0; q < MOE_STAGE_N; ++q) {
        t->used[q] = 0;
        t->ev[q] = nullptr;
    }
    for (int q = 0; q < MOE_STAGE_N; ++q) {
        t->ev[q] = new (std::nothrow) hipEvent_t[2 * (size_t)capacity]();
        if (!t->ev[q]) {
            moe_timer_destroy(t);
            return MOE_EINVAL;
        }
        for (int j = 0; j < 2 * capacity; ++j)
            if (hipEventCreate(&t->ev[q][j]) != hipSuccess) {
                t->ev[q][j] = nullptr;
                moe_timer_destroy(t);
                return MOE_EHIP;
            }
    }
    *out = t;
    return MOE_OK;
}

int moe_timer_destroy(moe_timer_t *t)
{
    if (!t) return MOE_EINVAL;
    for (int q = 0; q < MOE_STAGE_N; ++q) {
        if (!t->ev[q]) continue;
        for (int j = 0; j < 2 * t->capacity; ++j)
            if (t->ev[q][j]) (void)hipEventDestroy(t->ev[q][j]);
        delete[] t->ev[q];
    }
    delete t;
    return MOE_OK;
}

int moe_timer_read(moe_timer_t *t, double *total_ms, int64_t *launches)
{
    if (!t || !total_ms || !launches) return MOE_EINVAL;
    int rc = MOE_OK;
    for (int q = 0; q < MOE_STAGE_N; ++q) {
        double sum = 0.0;
        for (int j = 0; j < t->used[q]; ++j) {
            float ms = 0.f;
            if (hipEventSynchronize(t->ev[q][2 * j + 1]) != hipSuccess ||
                hipEventElapsedTime(&ms, t->ev[q][2 * j], t->ev[q][2 * j + 1]) != hipSuccess) {
                rc = MOE_EHIP;
                continue;
            }
            sum += ms;
        }
        total_ms[q] += sum;
        launches[q] += t->used[q];
        t->used[q] = 0;
    }
    return rc;
}

const char *moe_status_str(int status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported by this build";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_ENOSPACE: return "request larger than the fixed buffer of the allocation-free call";
    default: return "unknown status";
    }
}

}  // extern "C"
