"""The five synthetic workloads (shapes, width schedules, M values, seeds).

Synthetic stand-ins for the pages' Llama-3-70B runs (ainews.cool exllamav3
article, benchmark table; promptquorum.com "ExLlamaV2 explained": a 70B model
in 24 GB at about 2.55 bits per weight), which need trained weights and
datasets.  Every tensor is seeded per (config, linear, tensor).

  cfg1  one 4096 -> 4096 layer, uniform 4-bit, M = 1
  cfg2  one 8192 -> 8192 layer, mixed 2.55 bpw, M in {1, 4, 8, 16}
  cfg3  one 70B decoder block (7 linears), mixed 2.55 bpw, M = 1
  cfg4  the same 7 shapes, mixed 4.0 bpw from {3,4,5,6}, M = 2048 (prefill)
  cfg5  80 such blocks (560 linears), mixed 2.55 bpw, M = 1 and 16
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import BLOCK_SHAPES, GROUP, N_BLOCKS_70B, activations, layer_widths, seed_for, weight


@dataclass(frozen=True)
class LinearSpec:
    config: int
    index: int          # linear index within the config
    name: str
    K: int
    N: int
    kind: str           # width schedule: "u4", "mixed2.55", "mixed4.0"

    @property
    def G(self) -> int:
        return self.K // GROUP

    def w_seed(self) -> int:
        return seed_for("exq", self.config, self.index, "W")

    def sched_seed(self) -> int:
        return seed_for("exq", self.config, self.index, "widths")

    def x_seed(self, M: int) -> int:
        return seed_for("exq", self.config, self.index, "x", M)


def linears(config: int) -> list[LinearSpec]:
    if config == 1:
        return [LinearSpec(1, 0, "single", 4096, 4096, "u4")]
    if config == 2:
        return [LinearSpec(2, 0, "single", 8192, 8192, "mixed2.55")]
    if config == 3:
        return [LinearSpec(3, i, n, K, N, "mixed2.55") for i, (n, K, N) in enumerate(BLOCK_SHAPES)]
    if config == 4:
        return [LinearSpec(4, i, n, K, N, "mixed4.0") for i, (n, K, N) in enumerate(BLOCK_SHAPES)]
    if config == 5:
        out = []
        for blk in range(N_BLOCKS_70B):
            for j, (n, K, N) in enumerate(BLOCK_SHAPES):
                out.append(LinearSpec(5, blk * len(BLOCK_SHAPES) + j, "b%d.%s" % (blk, n), K, N, "mixed2.55"))
        return out
    raise ValueError(config)


M_VALUES = {1: (1,), 2: (1, 4, 8, 16), 3: (1,), 4: (2048,), 5: (1, 16)}


def make_weight(spec: LinearSpec, out: np.ndarray | None = None) -> np.ndarray:
    return weight(spec.w_seed(), spec.N, spec.K, 0.02, out=out)


def make_widths(spec: LinearSpec, W: np.ndarray | None = None) -> np.ndarray:
    return layer_widths(spec.kind, spec.G, spec.sched_seed(), W)


def make_x(spec: LinearSpec, M: int) -> np.ndarray:
    return activations(spec.x_seed(M), M, spec.K)


def algorithmic_bytes(K: int, N: int, widths, M: int) -> int:
    """Codes + fp16 scales + per-group metadata + fp16 x + fp16 y."""
    G = K // GROUP
    codes = int(np.asarray(widths, dtype=np.int64).sum()) * 16 * N
    return codes + 2 * G * N + 5 * G + 2 * M * K + 2 * M * N
