"""Seeded synthetic inputs for the MoE layer forward.

This module only draws random numbers and shapes them into the layer's
inputs (router logits, token activations, expert weights). It holds none of
the layer's arithmetic, so the HIP path and the CPU oracle can both be fed
from it without sharing any computation.

Recipe (one numpy PCG64 stream per workload, seed 0 unless stated):
  z      = standard_normal((T, E), float32)         router logits ~ N(0, 1)
  b_e    = skew bias, computed in float64, rounded to float32
  logits = z + b                                     float32 add
  x      = standard_normal((T, d_model), float32)    then rounded to dtype
  for e in 0..E-1, in order:
      Wg[e] = standard_normal((d_ff, d_model)) * float32(1/sqrt(d_model))
      Wu[e] = standard_normal((d_ff, d_model)) * float32(1/sqrt(d_model))
      Wd[e] = standard_normal((d_model, d_ff)) * float32(1/sqrt(d_ff))
  each rounded to dtype (bf16 by round-to-nearest-even).

Arrays are returned as float32 holding values that are exact in the
workload's dtype, so a bf16 device copy is an exact conversion.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterator

import numpy as np

from .configs import Workload


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), in place
    semantics on a copy; returns float32 holding bf16-exact values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) \
        & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def skew_bias(w: Workload) -> np.ndarray:
    """Per-expert logit bias b (float32 [E]) that shapes the routing load."""
    kind = w.skew[0]
    b = np.zeros(w.E, dtype=np.float64)
    if kind == "none":
        pass
    elif kind == "zipf":
        s = float(w.skew[1])
        b = s * np.log(1.0 / (np.arange(w.E, dtype=np.float64) + 1.0))
    elif kind == "hot":
        e0, val = int(w.skew[1]), float(w.skew[2])
        b[e0] = val
    else:
        raise ValueError(f"unknown skew {w.skew!r}")
    return b.astype(np.float32)


@dataclasses.dataclass
class Activations:
    logits: np.ndarray  # float32 [T, E]
    x: np.ndarray       # float32 [T, d_model], dtype-exact


class Stream:
    """The workload's random stream, consumed in recipe order."""

    def __init__(self, w: Workload):
        self.w = w
        self.rng = np.random.Generator(np.random.PCG64(w.seed))
        self._stage = 0

    def activations(self) -> Activations:
        assert self._stage == 0, "activations must be drawn first"
        w = self.w
        z = self.rng.standard_normal((w.T, w.E), dtype=np.float32)
        logits = (z + skew_bias(w)[None, :]).astype(np.float32)
        x = _to_dtype(self.rng.standard_normal((w.T, w.d_model),
                                               dtype=np.float32), w.dtype)
        self._stage = 1
        return Activations(logits=np.ascontiguousarray(logits), x=x)

    def expert_weights(self) -> Iterator[tuple]:
        """Yield (e, Wg_e [f,d], Wu_e [f,d], Wd_e [d,f]) for e = 0..E-1."""
        assert self._stage == 1, "draw activations before weights"
        w = self.w
        sd = np.float32(1.0 / math.sqrt(w.d_model))
        sf = np.float32(1.0 / math.sqrt(w.d_ff))
        for e in range(w.E):
            g = self.rng.standard_normal((w.d_ff, w.d_model), dtype=np.float32)
            g *= sd
            u = self.rng.standard_normal((w.d_ff, w.d_model), dtype=np.float32)
            u *= sd
            dn = self.rng.standard_normal((w.d_model, w.d_ff), dtype=np.float32)
            dn *= sf
            yield e, _to_dtype(g, w.dtype), _to_dtype(u, w.dtype), \
                _to_dtype(dn, w.dtype)
        self._stage = 2


@dataclasses.dataclass
class Inputs:
    logits: np.ndarray  # [T, E] float32
    x: np.ndarray       # [T, d] float32 (dtype-exact)
    Wg: np.ndarray      # [E, f, d]
    Wu: np.ndarray      # [E, f, d]
    Wd: np.ndarray      # [E, d, f]


def generate(w: Workload) -> Inputs:
    """All inputs of a workload as host float32 arrays (dtype-exact values)."""
    s = Stream(w)
    act = s.activations()
    Wg = np.empty((w.E, w.d_ff, w.d_model), dtype=np.float32)
    Wu = np.empty((w.E, w.d_ff, w.d_model), dtype=np.float32)
    Wd = np.empty((w.E, w.d_model, w.d_ff), dtype=np.float32)
    for e, g, u, dn in s.expert_weights():
        Wg[e], Wu[e], Wd[e] = g, u, dn
    return Inputs(act.logits, act.x, Wg, Wu, Wd)


def generate_activations(w: Workload) -> Activations:
    return Stream(w).activations()
