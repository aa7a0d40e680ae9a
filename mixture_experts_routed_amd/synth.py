"""Seeded synthetic inputs for the routed MoE layer.

This module only draws inputs: router logits and the router's top-k choice,
token activations and expert weights. It holds none of the layer's own
arithmetic (plan, gather, expert FFN, combine), so that both the HIP path and
the CPU oracle can take their inputs from here without sharing any code of
the method.

The pages measure real models with trained, quantised experts. Those weights
are not available, so every workload here is synthetic with the pages' shapes
and routing statistics:

* prefill layer, 512 experts, top-10, tm=16 (Round 4 Track C: Prefill MoE
  Plan ... audit, Table 2.1 and Table 2.2: T up to 2048, hidden size 2560);
* 44-100% of 256 experts touched by one 512-token ubatch (Add --moe-mode
  sweep-prefill ..., Motivation);
* a handful of tokens routed top-8, M of about 1 per expert (Batched resident
  MoE experts on Apple Silicon ..., Contribution);
* a 32K prompt processed in 2048-token chunks (#372 Prompt path ..., Speed);
* the prefill shape with tail skipping: a token's lowest-weight top-k slots
  routed to no expert (id -1), as in the plan's parity runs (Round 4 Track C
  audit, section 3). The pages do not give the skipping rule; here a slot is
  skipped when its renormalised weight is below 0.75/K (about 23% of the slots
  at this shape; the top-1 slot is never skipped).

Every random stream is numpy PCG64 seeded by SeedSequence([seed, tag, e]), so
any single expert's weights can be regenerated on their own.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

# stream tags: one independent random stream per kind of input
TAG_LOGITS, TAG_BIAS, TAG_X, TAG_WG, TAG_WU, TAG_WD, TAG_PERM, TAG_Y = range(8)

DTYPES = ("f32", "f16", "bf16")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class Config:
    """One MoE layer workload. Weights: W_gate, W_up [E, d, f]; W_down [E, f, d]."""

    name: str
    T: int          # tokens in the workload
    d: int          # hidden size
    E: int          # experts
    K: int          # experts per token (top-k)
    f: int          # expert FFN intermediate size
    dtype: str      # activation and weight element type: f32 | f16 | bf16
    tm: int = 16    # row padding: each expert's row count is rounded up to tm
    chunk: int = 0  # tokens per layer call (0: all T in one call)
    bias: str = "none"  # per-expert router bias: none | normal0.5 | zipf1.1
    tail_skip: float = 0.0  # slots with weight < tail_skip / K get id -1
    x_std: float = 0.02
    w_std: float = 0.02
    seed: int = 0

    @property
    def tokens_per_call(self) -> int:
        return self.chunk if self.chunk else self.T

    @property
    def ncalls(self) -> int:
        return self.T // self.tokens_per_call


CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", T=64, d=128, E=8, K=2, f=256, dtype="f32", seed=1001),
    "prefill_fp16": Config("prefill_fp16", T=2048, d=2560, E=512, K=10, f=768, dtype="f16", seed=1002),
    "decode_bf16": Config("decode_bf16", T=4, d=2816, E=128, K=8, f=704, dtype="bf16", seed=1003),
    "ubatch_bf16": Config("ubatch_bf16", T=512, d=4096, E=256, K=8, f=2048, dtype="bf16",
                          bias="normal0.5", seed=1004),
    "long_skewed_fp16": Config("long_skewed_fp16", T=32768, d=2560, E=512, K=10, f=768, dtype="f16",
                               chunk=2048, bias="zipf1.1", seed=1005),
    "prefill_tailskip_fp16": Config("prefill_tailskip_fp16", T=2048, d=2560, E=512, K=10, f=768,
                                    dtype="f16", tail_skip=0.75, seed=1006),
    # the long prompt's inputs (same seed and bias) planned as one call: the
    # heaviest experts get ~32K rows, so the grouped GEMMs reach the matrix cores' bound
    "long_onepass_fp16": Config("long_onepass_fp16", T=32768, d=2560, E=512, K=10, f=768,
                                dtype="f16", bias="zipf1.1", seed=1005),
}
CONFIG_ORDER = list(CONFIGS)


def rng(seed: int, tag: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, sub])))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_dtype(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the element type (nearest-even) and return raw storage.

    f32 -> float32 array; f16 / bf16 -> uint16 bit patterns.
    """
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f32":
        return a32
    if dtype == "f16":
        return a32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        return torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def router_bias(cfg: Config) -> np.ndarray:
    """Per-expert additive router bias (fp64, [E])."""
    if cfg.bias == "none":
        return np.zeros(cfg.E)
    if cfg.bias == "normal0.5":
        return rng(cfg.seed, TAG_BIAS).standard_normal(cfg.E) * 0.5
    if cfg.bias == "zipf1.1":
        # softmax(bias) is a Zipf(s=1.1) law over a seeded ranking of the experts
        rank = rng(cfg.seed, TAG_PERM).permutation(cfg.E) + 1
        return -1.1 * np.log(rank.astype(np.float64))
    raise ValueError(cfg.bias)


def routing(cfg: Config, T: int | None = None):
    """Router output for all T tokens: ids int32 [T, K], weights fp32 [T, K].

    logits = N(0,1) + bias (fp64); softmax over the E experts; the K largest
    probabilities in descending order (ties to the lower expert id) are kept
    and renormalised to sum to one. Column k of ids is the k-th choice. With
    tail skipping, slots whose weight is below tail_skip / K get id -1 (their
    weight is left in w; a skipped slot contributes nothing).
    """
    T = cfg.T if T is None else T
    logits = rng(cfg.seed, TAG_LOGITS).standard_normal((T, cfg.E)) + router_bias(cfg)[None, :]
    order = np.argsort(-logits, axis=1, kind="stable")[:, : cfg.K]
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    pk = np.take_along_axis(p, order, axis=1)
    w = (pk / pk.sum(axis=1, keepdims=True)).astype(np.float32)
    ids = order.astype(np.int32)
    if cfg.tail_skip > 0:
        ids[w < np.float32(cfg.tail_skip / cfg.K)] = -1
    return ids, w


def router_logits(cfg: Config, T: int | None = None) -> np.ndarray:
    """Router logits as the router GEMM would hand them over: fp32 [T, E]
    (N(0,1) + the config's per-expert bias, rounded from fp64)."""
    T = cfg.T if T is None else T
    logits = rng(cfg.seed, TAG_LOGITS).standard_normal((T, cfg.E)) + router_bias(cfg)[None, :]
    return logits.astype(np.float32)


def activations(cfg: Config, T: int | None = None) -> np.ndarray:
    """Token activations x [T, d] in the config's element type (raw storage)."""
    T = cfg.T if T is None else T
    x = rng(cfg.seed, TAG_X).standard_normal((T, cfg.d), dtype=np.float32) * np.float32(cfg.x_std)
    return to_dtype(x, cfg.dtype)


def _weight_shape(cfg: Config, which: str):
    return (cfg.d, cfg.f) if which in ("gate", "up") else (cfg.f, cfg.d)


_WTAG = {"gate": TAG_WG, "up": TAG_WU, "down": TAG_WD}


def expert_weight(cfg: Config, which: str, e: int) -> np.ndarray:
    """One expert's matrix: gate/up [d, f], down [f, d], raw storage."""
    shape = _weight_shape(cfg, which)
    a = rng(cfg.seed, _WTAG[which], e).standard_normal(shape[0] * shape[1], dtype=np.float32)
    a *= np.float32(cfg.w_std)
    return to_dtype(a, cfg.dtype).reshape(shape)


def expert_weights(cfg: Config, which: str, experts=None) -> np.ndarray:
    """Stacked expert matrices [len(experts), *shape] (all experts by default)."""
    experts = list(range(cfg.E)) if experts is None else list(experts)
    shape = _weight_shape(cfg, which)
    out = np.empty((len(experts),) + shape, dtype=storage_dtype(cfg.dtype))

    def fill(j):
        out[j] = expert_weight(cfg, which, experts[j])

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(len(experts))))
    return out


def random_rows(seed: int, nrows: int, ncols: int, std: float = 1.0) -> np.ndarray:
    """fp32 rows N(0, std) (used as a stand-alone expert-output input)."""
    return rng(seed, TAG_Y).standard_normal((nrows, ncols), dtype=np.float32) * np.float32(std)


def random_ids(seed: int, T: int, K: int, E: int, p_skip: float = 0.0, p_bad: float = 0.0,
               dup: bool = True) -> np.ndarray:
    """Arbitrary (not router-shaped) ids for plan fuzzing: duplicates within a
    token allowed, a fraction set to -1 (skipped) and a fraction out of range."""
    g = rng(seed, TAG_LOGITS, 7)
    ids = g.integers(0, E, size=(T, K), dtype=np.int64)
    if not dup:
        ids = np.stack([g.permutation(E)[:K] for _ in range(T)])
    u = g.random((T, K))
    ids[u < p_skip] = -1
    bad = (u >= p_skip) & (u < p_skip + p_bad)
    badv = g.integers(E, E + 1000, size=(T, K))
    badv[g.random((T, K)) < 0.5] *= -1
    badv[badv == -1] = -2
    ids[bad] = badv[bad]
    return ids.astype(np.int32)
