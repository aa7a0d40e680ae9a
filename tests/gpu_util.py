"""Helpers of the GPU parity tests: seeded inputs on host and device, and the
comparison measures. Inputs come from mixture_experts_routed_amd.synth (the
seeded generator) or from the oracle -- never from the HIP path."""
from __future__ import annotations

import sys
from dataclasses import dataclass, field, replace

import numpy as np
import torch

from mixture_experts_routed_amd import abi, synth

TORCH16 = {"f16": torch.float16, "bf16": torch.bfloat16}
TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 5e-3}  # max|gpu - ref| / max|ref|
POLLUTE = 0xDEADBEEF - (1 << 32)  # as int32


def say(*a):
    """name the case before a GPU step (flushed, so it survives a crash)"""
    print(*a, file=sys.stderr, flush=True)


def dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """host array (raw storage) -> GPU tensor; uint16 arrays become f16/bf16"""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(TORCH16[dtype])
    else:
        t = torch.from_numpy(a)
    return t.to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> host raw storage (f16/bf16 as uint16 bit patterns)"""
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def polluted(n: int, dtype=torch.int32) -> torch.Tensor:
    t = torch.full((max(int(n), 1),), POLLUTE, dtype=torch.int32, device="cuda")
    return t.view(dtype) if dtype != torch.int32 else t


@dataclass
class Case:
    cfg: synth.Config
    ids: np.ndarray
    w: np.ndarray
    x: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    _dev: dict = field(default_factory=dict)

    def d(self, name: str) -> torch.Tensor:
        if name not in self._dev:
            a = getattr(self, name)
            self._dev[name] = dev(a, self.cfg.dtype)
        return self._dev[name]

    def drop_device(self):
        self._dev.clear()
        torch.cuda.empty_cache()


def make_case(cfg: synth.Config) -> Case:
    ids, w = synth.routing(cfg)
    return Case(cfg, ids, w, synth.activations(cfg), synth.expert_weights(cfg, "gate"),
                synth.expert_weights(cfg, "up"), synth.expert_weights(cfg, "down"))


def custom(name, T, d, E, K, f, dtype, tm=16, bias="none", seed=7, x_std=0.02, w_std=0.02):
    return synth.Config(name, T=T, d=d, E=E, K=K, f=f, dtype=dtype, tm=tm, bias=bias, seed=seed,
                        x_std=x_std, w_std=w_std)


def chunk_of(case: Case, c: int):
    """ids, w, x of layer call c (token chunk c)"""
    Tc = case.cfg.tokens_per_call
    sl = slice(c * Tc, (c + 1) * Tc)
    return case.ids[sl], case.w[sl], case.x[sl]


__all__ = ["abi", "synth", "replace", "Case", "make_case", "custom", "dev", "host", "rel_err",
           "polluted", "say", "TOL", "chunk_of"]
