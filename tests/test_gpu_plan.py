"""GPU parity of moe_plan: every output bit-exact against the oracle's counting
sort, with the output buffers pre-polluted (0xDEADBEEF) so that an element the
kernels fail to write is caught, and rows beyond nr checked untouched."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import POLLUTE, abi, host, polluted, say, synth

pytestmark = pytest.mark.gpu


def run_plan(ids: np.ndarray, w: np.ndarray, E: int, tm: int):
    T, K = ids.shape
    z = abi.moe_plan_sizes(T, K, E, tm)
    o = dict(cnt=polluted(E), eoff=polluted(E + 1), tiles=polluted(z.max_tiles),
             stok=polluted(z.max_rows), sw=polluted(z.max_rows, torch.float32),
             pos=polluted(T * K), boff=polluted(z.nblk * E), meta=polluted(abi.META_N))
    scratch = torch.full((max(z.scratch_bytes // 4, 1),), 777777, dtype=torch.int32, device="cuda")
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda()
    w_d = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    abi.moe_plan(ids_d, w_d, T, K, E, tm, o["cnt"], o["eoff"], o["tiles"], o["stok"], o["sw"],
                 o["pos"], o["boff"], o["meta"], scratch)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in o.items()}, z


def check_plan(ids, w, E, tm, label):
    say(f"[plan] {label}: T={ids.shape[0]} K={ids.shape[1]} E={E} tm={tm}")
    g, z = run_plan(ids, w, E, tm)
    r = oracle.plan(ids, w, E, tm, B=1024)
    nr, nt = int(r["meta"][2]), int(r["meta"][3])
    assert np.array_equal(g["meta"], r["meta"]), (g["meta"], r["meta"])
    assert np.array_equal(g["cnt"], r["cnt"])
    assert np.array_equal(g["eoff"], r["eoff"])
    assert np.array_equal(g["tiles"][:nt], r["tiles"])
    assert np.array_equal(g["stok"][:nr], r["stok"])
    assert np.array_equal(g["sw"][:nr].view(np.uint32), r["sw"].view(np.uint32))
    assert np.array_equal(g["pos"], r["pos"])
    assert np.array_equal(g["boff"][: r["boff"].size], r["boff"])
    # nothing written past the plan's rows / tiles
    assert np.all(g["stok"][nr:] == POLLUTE)
    assert np.all(g["sw"][nr:].view(np.int32) == POLLUTE)
    assert np.all(g["tiles"][nt:] == POLLUTE)
    return g


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_plan_bit_exact_configs(name):
    cfg = synth.CONFIGS[name]
    ids, w = synth.routing(cfg)
    Tc = cfg.tokens_per_call
    for c in range(cfg.ncalls):  # every 2048-token chunk of the long prompt
        sl = slice(c * Tc, (c + 1) * Tc)
        check_plan(ids[sl], w[sl], cfg.E, cfg.tm, f"{name} call {c}")


FUZZ = [
    # T, K, E, tm, p_skip, p_bad, seed
    (1, 1, 1, 16, 0.0, 0.0, 1),
    (1, 1, 1, 1, 0.0, 0.0, 2),
    (3, 5, 2, 1, 0.2, 0.2, 3),
    (100, 10, 512, 16, 0.1, 0.05, 4),
    (1000, 7, 1024, 16, 0.0, 0.0, 5),      # E at the limit, ragged last block
    (513, 2, 1024, 64, 0.3, 0.0, 6),
    (4096, 2, 2, 16, 0.0, 0.0, 7),         # 64 copies of one expert per wave
    (777, 9, 37, 5, 0.05, 0.05, 8),        # tm not a power of two
    (2048, 10, 512, 16, 0.25, 0.0, 9),     # tail-skipping shaped
    (4, 64, 64, 1, 0.0, 0.0, 10),          # K = E, duplicates allowed
    (200, 3, 1, 32, 0.5, 0.1, 11),         # one expert
    (6000, 8, 256, 16, 0.0, 0.0, 12),      # many blocks (three-launch path)
    (4096, 8, 512, 16, 0.02, 0.01, 13),    # 32 blocks: largest single-launch plan
    (32769, 1, 300, 16, 0.0, 0.0, 14),     # 33 blocks: smallest three-launch plan
    (16384, 4, 1000, 8, 0.05, 0.0, 15),    # 64 blocks
    # at most 64 entries: the one-wavefront plan
    (8, 8, 1024, 16, 0.1, 0.05, 16),       # 64 entries, E at the limit: 16 experts per lane
    (64, 1, 1, 48, 0.0, 0.0, 17),          # one expert: 96 padded rows, two work items
    (4, 16, 16, 1, 0.0, 0.0, 18),          # K = E, duplicates allowed
    (2, 32, 100, 64, 0.5, 0.0, 19),        # half skipped, tm 64
    (5, 13, 3, 7, 0.3, 0.3, 20),           # 65 entries: just past one wavefront
]


def random_plans(n=40, seed=4242):
    """seeded random plan shapes: both plan paths, any tile, skipped and bad ids"""
    g = np.random.default_rng(seed)
    out = []
    for k in range(n):
        E = int(g.choice([1, 2, 5, 31, 64, 65, 128, 300, 512, 777, 1000, 1024]))
        K = int(g.integers(1, 17))
        T = int(g.choice([1, 2, 7, 100, 1023, 1024, 1025, 3000, 4096, 9999, 20000, 40000]))
        T = max(1, min(T, 200_000 // K))
        tm = int(g.choice([1, 2, 3, 8, 16, 16, 31, 64]))
        ps, pb = float(g.choice([0.0, 0.0, 0.1, 0.5])), float(g.choice([0.0, 0.0, 0.02]))
        out.append((T, K, E, tm, ps, pb, 100 + k))
    return out


FUZZ += random_plans()


@pytest.mark.parametrize("T,K,E,tm,ps,pb,seed", FUZZ)
def test_plan_bit_exact_fuzz(T, K, E, tm, ps, pb, seed):
    ids = synth.random_ids(seed, T, K, E, p_skip=ps, p_bad=pb)
    w = synth.random_rows(seed, T, K)
    check_plan(ids, w, E, tm, f"fuzz seed {seed}")


@pytest.mark.parametrize("T", [50, 10], ids=["fused", "one_wavefront"])
def test_plan_all_skipped_and_all_bad(T):
    K, E = 4, 16
    ids = np.full((T, K), -1, np.int32)
    w = synth.random_rows(3, T, K)
    g = check_plan(ids, w, E, 16, "all skipped")
    assert g["meta"][2] == 0 and g["meta"][6] == T * K
    ids = np.full((T, K), E + 5, np.int32)
    g = check_plan(ids, w, E, 16, "all bad")
    assert g["meta"][7] == T * K


def test_plan_deterministic_and_repeatable():
    cfg = synth.CONFIGS["prefill_fp16"]
    ids, w = synth.routing(cfg)
    a, _ = run_plan(ids, w, cfg.E, cfg.tm)
    b, _ = run_plan(ids, w, cfg.E, cfg.tm)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
