"""A CPU model of the grouped FFN kernels' index arithmetic (no kernel runs):
for each workload and the seeded random shapes, the oracle's plan gives the
work list (the documented format), and every logical workgroup of each launch
is mapped the way the kernels map it -- XCD-contiguous block ranges, (item,
column group, K split), wide / tall / big cells -- to the byte ranges its
buffer descriptors cover and the rows and columns it stores. Each must lie
inside its buffer: the packed or row-major weight sets, x (gathered rows) or
xs, h, y and the split-K partial planes. The host's launch grids must cover
every logical block. The split counts and big-cell choice are taken from the
library's own host calls, so the model follows the sizes the library uses.

Shapes: the workloads (first layer call), the random sweep of the GPU tests,
and the hand-picked launch-path cases (split K, tall and big cells)."""
import numpy as np
import pytest

import oracle
from mixture_experts_routed_amd import abi, synth
from test_gpu_ffn import PATHS as FFN_PATHS
from test_gpu_ffn import worklist_model
from test_gpu_packed import BIG
from test_gpu_random_shapes import SHAPES

ITEM = 64  # rows per work item


def ceil(a, b):
    return -(-a // b)


def round8(v):
    return ceil(v, 8) * 8


def max_items(E, tm, R):
    return R // ITEM + 1 + min(E, ceil(R, tm))


def split_model(cells, Kd, kstep):
    """K splits and steps per split of a projection (the library's rule)"""
    nsteps = ceil(Kd, kstep)
    s = ceil(512, cells) if cells < 192 else 1
    s = min(s, 8)
    smax = max(nsteps // 8, 1)
    s = min(s, smax)
    per = ceil(nsteps, s)
    return ceil(nsteps, per), per


def packed_geom(Kd, N, gateup, es):
    m = 1 if gateup else 2
    kstep = 32 if es == 2 else 16
    return {"gs": ceil(N, 256 * m), "nst": ceil(Kd, kstep), "m": m, "step": 16384 * m}


class Buffers:
    """byte sizes of the buffers one projection reads and writes"""

    def __init__(self, cfg, R, T, gateup, packed, es):
        E, d, f = cfg.E, cfg.d, cfg.f
        Kd, N = (d, f) if gateup else (f, d)
        self.Kd, self.N, self.es = Kd, N, es
        if packed:
            self.B = abi.moe_packed_weight_bytes(E, d, f, abi.DTYPE_NAME[cfg.dtype],
                                                 abi.MOE_W_GATE_UP if gateup else abi.MOE_W_DOWN)
        else:
            self.B = E * Kd * N * es
        self.x = T * d * es
        self.xs = R * d * es
        self.h = R * f * es
        self.y = R * d * 4


def check_range(name, base, size, limit):
    assert 0 <= base and size >= 0 and base + size <= limit, (name, base, size, limit)
    assert size < 2 ** 32, (name, size)  # a descriptor's range is 32-bit


def model_projection(cfg, eoff, R, T, gateup, packed, gathered, nsplit, per, big, items, nfour):
    es = synth.ELEM_BYTES[cfg.dtype]
    kstep = 32 if es == 2 else 16
    b = Buffers(cfg, R, T, gateup, packed, es)
    Kd, N = b.Kd, b.N
    SW = 64 if gateup else 128  # columns per wave slice
    HALF = 0 if gateup else 64
    gs = ceil(N, 4 * SW)
    pg = packed_geom(Kd, N, gateup, es)
    if packed:
        assert pg["gs"] == gs
    E = cfg.E
    nitems = len(items)
    # scratch: counters, items, then the partial planes when split
    plane = R * (2 * N if gateup else N)
    # ---- 4-wavefront kernel ----
    ifirst = nfour if big else 0
    per_item = gs * nsplit
    nlogical = (nitems - ifirst) * per_item
    grid = round8(max_items(E, cfg.tm, R) * gs * nsplit)
    assert ceil(nlogical, 8) <= grid // 8, (nlogical, grid)  # xcd_logical_block covers all
    for lb in range(nlogical):
        il, rem = divmod(lb, per_item)
        i = ifirst + il
        g, split = divmod(rem, nsplit)
        kb = split * per * kstep
        ke = min(Kd, kb + per * kstep)
        assert kb < ke, (kb, ke)
        ex, row0, nrows, run = (int(v) for v in items[i])
        assert 0 <= ex < E and 0 < nrows <= ITEM and row0 + nrows <= R
        rl, j = run & 0xFF, (run >> 8) & 0xFF
        if rl in (4, 2) and j < rl and i >= j:
            R_, i0 = rl, i - j
            C = 4 // R_
            cells = [(items[i0 + q] if i0 + q < nitems and items[i0 + q][0] == ex else None)
                     for q in range(R_)]
            # producers: C slices x 2 streams of this group
            for pcs in range(C):
                pslice = 4 * g + C * j + pcs
                wp = C * j + pcs
                assert wp <= 3
                for pm in range(2):
                    if packed:
                        s0, s1 = kb // kstep, ceil(ke, kstep)
                        mm = 0 if gateup else pm
                        tb = (((((ex * pg["gs"] + g) * pg["nst"] + s0) * 4 + wp) * pg["m"] + mm)
                              * 4096)
                        span = (s1 - s0) * pg["step"]
                        rng = 0 if pslice * SW >= N else span - (wp * pg["m"] + mm) * 4096
                        check_range("tall B packed", tb, rng, b.B)
                    else:
                        wofs = (ex * Kd * N + kb * N) * es
                        kbytes = (ke - kb) * N * es
                        if pslice * SW < N:
                            base = wofs + (0 if gateup or pm == 0 else HALF * es)
                            rng = kbytes if gateup or pm == 0 else kbytes - HALF * es
                            check_range("tall B rowmajor", base, rng, b.B)
            for c in cells:
                if c is not None:
                    model_rows(c, b, gathered, Kd, es, T, R)
                    model_stores(c, b, gateup, (4 * g + C * j) * SW, C * SW, N, R, nsplit, split,
                                 plane, HALF)
        else:
            for w in range(4):
                slice_ = 4 * g + w
                slice_ok = slice_ * SW < N
                if packed:
                    s0, s1 = kb // kstep, ceil(ke, kstep)
                    tb = ((((ex * pg["gs"] + g) * pg["nst"] + s0) * 4 + w) * pg["m"]) * 4096
                    span = (s1 - s0) * pg["step"]
                    r0 = span - w * pg["m"] * 4096 if slice_ok else 0
                    check_range("wide B0 packed", tb, r0, b.B)
                    if not gateup:
                        r1 = span - (w * pg["m"] + pg["m"] - 1) * 4096 if slice_ok else 0
                        check_range("wide B1 packed", tb + 4096, r1, b.B)
                elif slice_ok:
                    wofs = (ex * Kd * N + kb * N) * es
                    kbytes = (ke - kb) * N * es
                    check_range("wide B0 rowmajor", wofs, kbytes, b.B)
                    if not gateup:
                        assert kbytes >= HALF * es
                        check_range("wide B1 rowmajor", wofs + HALF * es, kbytes - HALF * es, b.B)
            model_rows(items[i], b, gathered, Kd, es, T, R)
            model_stores(items[i], b, gateup, 4 * g * SW, 4 * SW, N, R, nsplit, split, plane, HALF)
    # ---- 8-wavefront big cells ----
    if big:
        BCOLS = 128 if gateup else 256
        ncb = ceil(N, BCOLS)
        nquads = nfour // 4
        grid_big = round8((R // (3 * ITEM + 1)) * ncb)
        assert ceil(nquads * ncb, 8) <= grid_big // 8, (nquads, ncb, grid_big)
        for qd in range(nquads):
            run = items[4 * qd: 4 * qd + 4]
            ex, row0 = int(run[0][0]), int(run[0][1])
            assert all(int(r[0]) == ex for r in run)
            assert [int(r[3]) for r in run] == [4 | (q << 8) for q in range(4)]
            nvalid = int(run[3][1]) + int(run[3][2]) - row0
            assert 0 < nvalid <= 4 * ITEM and row0 + nvalid <= R
            for cb in range(ncb):
                gbase = (ex * pg["gs"] + (cb >> 1)) * pg["nst"] * pg["step"]
                check_range("big B", gbase, pg["nst"] * pg["step"], b.B)
                if gathered:
                    check_range("big A (x)", 0, b.x, b.x)
                else:
                    check_range("big A", row0 * Kd * es, nvalid * Kd * es,
                                b.xs if gateup else b.h)
                for r in run:
                    model_stores(r, b, gateup, cb * BCOLS, BCOLS, N, R, 1, 0, plane, 0)
    return nlogical


def model_rows(it, b, gathered, Kd, es, T, R):
    """the item's A rows: x through stok (gathered) or its rows of xs / h"""
    ex, row0, nrows, _ = (int(v) for v in it)
    if gathered:
        assert b.x < 2 ** 31  # the host gathers first otherwise
        check_range("A x", 0, b.x, b.x)
    else:
        check_range("A rows", row0 * Kd * es, nrows * Kd * es, R * Kd * es)


def model_stores(it, b, gateup, col0, ncols, N, R, nsplit, split, plane, HALF):
    """the item's stores in columns [col0, col0 + ncols) of its rows"""
    ex, row0, nrows, _ = (int(v) for v in it)
    assert row0 + nrows <= R
    cols = [c for c in range(col0, col0 + ncols, 4) if c < N]
    for c in cols:
        assert c + 4 <= N  # 4 columns per store, N a multiple of 8
    if nsplit > 1:
        last = (split * plane + (row0 + nrows - 1) * (2 * N if gateup else N) + N
                + (N if gateup else 0))
        assert last <= nsplit * plane
    elif gateup:
        check_range("h rows", row0 * N * b.es, nrows * N * b.es, b.h)
    else:
        check_range("y rows", row0 * N * 4, nrows * N * 4, b.y)


def plan_items(cfg, T, ids, w, R, runs_first):
    p = oracle.plan(ids, w, cfg.E, cfg.tm)
    items, nfour, _ = worklist_model(p["eoff"], cfg.E, R, runs_first)
    return p, items, nfour


CASES = ([synth.CONFIGS[n] for n in synth.CONFIG_ORDER] + SHAPES + [c[0] for c in FFN_PATHS]
         + BIG)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_gemm_launches_stay_in_bounds(cfg):
    T = cfg.tokens_per_call
    ids, w = synth.routing(cfg, T)
    dt = abi.DTYPE_NAME[cfg.dtype]
    es = synth.ELEM_BYTES[cfg.dtype]
    kstep = 32 if es == 2 else 16
    R = abi.moe_plan_sizes(T, cfg.K, cfg.E, cfg.tm).max_rows
    sgu, sdn = abi.moe_ffn_splits(cfg.E, cfg.d, cfg.f, cfg.tm, R, dt)
    mi = max_items(cfg.E, cfg.tm, R)
    # the model's split rule reproduces the library's
    ngu, per_gu = split_model(mi * ceil(cfg.f, 256), cfg.d, kstep)
    ndn, per_dn = split_model(mi * ceil(cfg.d, 512), cfg.f, kstep)
    assert (ngu, ndn) == (sgu, sdn)
    bigbits = abi.moe_ffn_big_cells(cfg.E, cfg.d, cfg.f, cfg.tm, R, dt)
    gathered = T * cfg.d * es < 2 ** 31
    for packed in (False, True):
        big_gu = packed and es == 2 and bool(bigbits & 1)
        big_dn = packed and es == 2 and bool(bigbits & 2)
        p, items, nfour = plan_items(cfg, T, ids, w, R, packed and (big_gu or big_dn))
        assert len(items) <= mi
        n = model_projection(cfg, p["eoff"], R, T, True, packed, gathered, sgu, per_gu, big_gu,
                             items, nfour)
        n += model_projection(cfg, p["eoff"], R, T, False, packed, False, sdn, per_dn, big_dn,
                              items, nfour)
        assert n > 0 or len(items) == 0


def test_model_catches_an_undersized_grid():
    """the model is live: with the gate/up grid computed from one work item too few,
    the prefill shape's coverage check fails"""
    cfg = synth.CONFIGS["prefill_fp16"]
    ids, w = synth.routing(cfg)
    R = abi.moe_plan_sizes(cfg.T, cfg.K, cfg.E, cfg.tm).max_rows
    _, items, nfour = plan_items(cfg, cfg.T, ids, w, R, False)
    short = np.concatenate([items, items[-1:].repeat(max_items(cfg.E, cfg.tm, R) -
                                                     len(items) + 9, axis=0)])
    with pytest.raises(AssertionError):
        model_projection(cfg, None, R, cfg.T, True, True, True, 1, 80, False, short, 0)


GATHER_WAVES = 2  # kGatherWaves of the gather kernel


def test_gather_model_matches_the_kernel_constant():
    """the partition model below uses the kernel's workgroup size"""
    import re
    from pathlib import Path
    src = (Path(__file__).resolve().parents[1] / "mixture_experts_routed_amd" / "csrc" /
           "gather_combine.hip").read_text()
    assert int(re.search(r"constexpr int kGatherWaves = (\d+);", src).group(1)) == GATHER_WAVES


GATHER_CASES = [synth.CONFIGS[n] for n in ("prefill_fp16", "decode_bf16", "tiny_fp32",
                                           "prefill_tailskip_fp16")] + SHAPES[:24]


@pytest.mark.parametrize("cfg", GATHER_CASES, ids=[c.name for c in GATHER_CASES])
def test_gather_partition_copies_every_row_once_in_bounds(cfg):
    """the standalone gather's grid (row groups of GATHER_WAVES x 64 rows, 8
    workgroups per group, one per XCD) and its ownership rule (token mod 8, a pad row by row mod 8)
    copy every row below nr exactly once, read only token rows below T and write
    only rows below nr"""
    T = cfg.tokens_per_call
    ids, w = synth.routing(cfg, T)
    R = abi.moe_plan_sizes(T, cfg.K, cfg.E, cfg.tm).max_rows
    p = oracle.plan(ids, w, cfg.E, cfg.tm)
    nr = len(p["stok"])
    stok = np.full(R, -1, np.int64)
    stok[:nr] = p["stok"]
    blocks = ceil(R, GATHER_WAVES * 64) * 8
    copies = np.zeros(nr, np.int64)
    for b in range(blocks):
        for wave in range(GATHER_WAVES):
            r0 = ((b >> 3) * GATHER_WAVES + wave) * 64
            if r0 >= nr:
                continue
            r = np.arange(r0, r0 + 64)
            ok = r < nr
            t = np.where(ok, stok[np.minimum(r, R - 1)], -1)
            owner = np.where((t >= 0) & (t < T), t & 7, r & 7)
            mine = r[ok & (owner == (b & 7))]
            assert np.all(mine < nr)
            tt = stok[mine]
            assert np.all((tt < T))  # tokens read are rows of x (pads read nothing)
            copies[mine] += 1
    assert np.all(copies == 1)


def wave_item_model(ids, E, K, tm, max_rows):
    """The gate/up launch's own work items for a call of at most 64 entries
    (wave_plan_item, lane l = entry l): an entry is its expert's first when no
    earlier entry has its id; item j is the j-th such expert by id, its rows
    start after the padded rows of the experts below it; its row r holds the
    token of the expert's r-th entry. Returns items [n, 4] and the tokens."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    valid = [0 <= e < E for e in flat]
    count = {}
    for e, v in zip(flat, valid):
        if v:
            count[e] = count.get(e, 0) + 1
    firsts = sorted(count)
    rows = {e: ceil(count[e], tm) * tm for e in firsts}
    items, toks = [], []
    for e in firsts:
        below = sum(rows[x] for x in firsts if x < e)
        items.append((e, below, min(ITEM, rows[e], max_rows - below), 1))
        t = [l // K for l, (x, v) in enumerate(zip(flat, valid)) if v and x == e]
        toks.append(t + [-1] * (ITEM - len(t)))
    return np.array(items, np.int32).reshape(-1, 4), toks


WAVE_CASES = [(4, 8, 128, 16, 0.0, 0.0, 1), (1, 1, 1, 16, 0.0, 0.0, 2),
              (8, 8, 1024, 16, 0.1, 0.05, 3), (16, 4, 4, 1, 0.0, 0.0, 4),
              (2, 32, 100, 64, 0.5, 0.0, 5), (64, 1, 1, 64, 0.0, 0.0, 6),
              (3, 16, 16, 8, 0.2, 0.2, 7), (5, 2, 8, 32, 1.0, 0.0, 8), (32, 2, 3, 2, 0.0, 0.3, 9)]


@pytest.mark.parametrize("T,K,E,tm,ps,pb,seed", WAVE_CASES)
def test_in_launch_items_are_the_work_list(T, K, E, tm, ps, pb, seed):
    """the items the gate/up launch derives itself (calls of at most 64 entries,
    tm dividing 64) are the documented work list of the oracle's plan, one single
    item per routed expert, and their token rows are the plan's stok"""
    assert T * K <= 64 and 64 % tm == 0
    ids = synth.random_ids(seed, T, K, E, p_skip=ps, p_bad=pb)
    w = synth.random_rows(seed, T, K)
    R = abi.moe_plan_sizes(T, K, E, tm).max_rows
    p = oracle.plan(ids, w, E, tm)
    want, _, runs = worklist_model(p["eoff"], E, R, runs_first=False)
    got, toks = wave_item_model(ids, E, K, tm, R)
    assert runs == 0 and np.array_equal(got, want)
    for (e, r0, nr, _), t in zip(got, toks):
        assert list(p["stok"][r0:r0 + nr]) == t[:nr]
