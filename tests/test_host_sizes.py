"""Host-side sizes against what the layer writes (CPU only, no kernel runs): for
the workloads and the seeded random shapes of test_gpu_random_shapes, with the
oracle's plan of their routing,
  * the plan bound (moe_plan_sizes.max_rows) covers the plan's padded rows;
  * moe_ffn_scratch_bytes covers the work list (256 bytes of counters, then
    16 bytes per item: each expert's padded rows cut into items of 64) and,
    when moe_ffn_splits says a projection is split, its fp32 partial planes
    (split x max_rows x 2f for gate/up, split x max_rows x d for down; the two
    projections share the region), the work list rounded up to 256 bytes;
  * moe_forward_layout carves every intermediate, at its full bound, from the
    workspace moe_forward_workspace asks for, without overlaps; for 16-bit
    layers the compact expert outputs (binary16 rows and their block
    exponents) fit in the y region."""
import numpy as np
import pytest

import oracle
from mixture_experts_routed_amd import abi, synth
from test_gpu_random_shapes import SHAPES

CASES = [synth.CONFIGS[n] for n in synth.CONFIG_ORDER] + SHAPES


def round256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_sizes_cover_the_layer(cfg):
    T = cfg.tokens_per_call
    ids, w = synth.routing(cfg)
    dt = abi.DTYPE_NAME[cfg.dtype]
    es = synth.ELEM_BYTES[cfg.dtype]
    z = abi.moe_plan_sizes(T, cfg.K, cfg.E, cfg.tm)
    R = z.max_rows
    sgu, sdn = abi.moe_ffn_splits(cfg.E, cfg.d, cfg.f, cfg.tm, R, dt)
    scratch = abi.moe_ffn_scratch_bytes(cfg.E, cfg.d, cfg.f, cfg.tm, R, dt)
    parts = max(sgu * R * 2 * cfg.f * 4 if sgu > 1 else 0, sdn * R * cfg.d * 4 if sdn > 1 else 0)
    for c in range(min(cfg.ncalls, 3)):
        p = oracle.plan(ids[c * T:(c + 1) * T], w[c * T:(c + 1) * T], cfg.E, cfg.tm)
        eoff = np.asarray(p["eoff"], np.int64)
        assert eoff[-1] <= R
        nitems = int(((np.diff(eoff) + 63) // 64).sum())
        assert round256(256 + 16 * nitems) + parts <= scratch, (nitems, sgu, sdn, scratch)

    L = abi.moe_forward_layout(T, cfg.K, cfg.E, cfg.d, cfg.f, cfg.tm, dt)
    total = abi.moe_forward_workspace(T, cfg.K, cfg.E, cfg.d, cfg.f, cfg.tm, dt)
    assert L.total <= total
    E, nent = cfg.E, T * cfg.K
    need = {"cnt": E * 4, "eoff": (E + 1) * 4, "tiles": z.max_tiles * 4, "stok": R * 4,
            "sw": R * 4, "pos": nent * 4, "boff": z.nblk * E * 4, "meta": 11 * 4,
            "plan_scratch": z.scratch_bytes, "xs": R * cfg.d * es, "h": R * cfg.f * es,
            "y": R * cfg.d * 4, "ffn_scratch": scratch}
    if cfg.dtype != "f32":
        # 16-bit layers keep y compact: binary16 rows, then one exponent byte per
        # 128 columns, inside the fp32-sized region
        assert R * cfg.d * 2 + R * ((cfg.d + 127) // 128) <= need["y"]
    spans = sorted((getattr(L, k), getattr(L, k) + n, k) for k, n in need.items())
    for (a0, a1, ka), (b0, b1, kb) in zip(spans, spans[1:]):
        assert a1 <= b0, (ka, kb)
    assert spans[-1][1] <= L.total
    for a0, _, k in spans:
        assert a0 % 16 == 0, k  # data arrays are 16-byte aligned, index arrays at least 4
