"""Seeded synthetic workloads for the quantized linear layer.

This module holds the workload shapes, the per-layer precision plans and the
seeded bf16 input generators. Both the HIP path (tests, bench) and the CPU
oracle draw their inputs from here, so it contains none of the quantization
arithmetic: only shapes, seeds and random draws.

The layer set (Q, K, V, O, Gate, Up, Down) is the set of linear layers of a
Llama-like block [SNIP, Fig. 4]. Every tensor is drawn in fp32 from a numpy
PCG64 generator keyed by (workload id, layer index, role) and rounded to bf16
by round-to-nearest-even (torch's fp32->bf16 cast).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

# Format ids shared with the C ABI (include/snip.h).
BF16, FP8, NVFP4, MXFP4 = 0, 1, 2, 3
FORMAT_NAMES = {BF16: "bf16", FP8: "fp8_e4m3", NVFP4: "nvfp4", MXFP4: "mxfp4"}

# Roles of the three bf16 tensors of a linear layer.
ROLE_X, ROLE_W, ROLE_DY = 0, 1, 2

LAYER_NAMES = ["Q", "K", "V", "O", "Gate", "Up", "Down"]


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    d_in: int
    d_out: int


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int                 # seed namespace
    name: str
    tokens: int              # T
    layers: tuple            # tuple[Layer]
    plan: tuple              # per-layer format id
    x_dist: str              # "normal", "normal_outliers", "student_t_cols"
    w_std: float = 0.02
    dy_std: float = 1e-3
    sr_seeds: tuple = (0,)

    def layer(self, name: str) -> Layer:
        for l in self.layers:
            if l.name == name:
                return l
        raise KeyError(name)


def _llama_layers(hidden: int, q_out: int, kv_out: int, ffn: int) -> tuple:
    return (
        Layer("Q", hidden, q_out),
        Layer("K", hidden, kv_out),
        Layer("V", hidden, kv_out),
        Layer("O", q_out, hidden),
        Layer("Gate", hidden, ffn),
        Layer("Up", hidden, ffn),
        Layer("Down", ffn, hidden),
    )


def random_plan(wid: int, n_layers: int, p_fp4: float = 0.5) -> tuple:
    """Per-layer FP8/NVFP4 choice, each layer NVFP4 with probability p_fp4.

    Drawn from its own seeded stream so the plan is reproducible and
    independent of the tensor data.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, 0xA11CE])))
    u = rng.random(n_layers)
    return tuple(NVFP4 if v < p_fp4 else FP8 for v in u)


def _make_workloads() -> Dict[str, Workload]:
    w = {}
    w["linear512"] = Workload(
        wid=1, name="linear512", tokens=256,
        layers=(Layer("L", 512, 512),), plan=(NVFP4,), x_dist="normal_outliers")
    tl = _llama_layers(2048, 2048, 256, 5632)
    w["tinyllama1b"] = Workload(
        wid=2, name="tinyllama1b", tokens=4096, layers=tl,
        plan=random_plan(2, len(tl)), x_dist="normal")
    l7 = _llama_layers(4096, 4096, 4096, 11008)
    # FP4 on Q, K, Gate, Up, Down and FP8 on V, O: the smallest per-layer FP4
    # FLOP share at or above 80 %.
    plan7 = tuple(FP8 if l.name in ("V", "O") else NVFP4 for l in l7)
    w["llama7b"] = Workload(
        wid=3, name="llama7b", tokens=8192, layers=l7, plan=plan7,
        x_dist="student_t_cols")
    l70 = _llama_layers(8192, 8192, 1024, 28672)
    w["llama70b"] = Workload(
        wid=4, name="llama70b", tokens=4096, layers=l70,
        plan=tuple(NVFP4 for _ in l70), x_dist="normal")
    w["down7b_sweep"] = Workload(
        wid=5, name="down7b_sweep", tokens=16384, layers=(Layer("Down", 11008, 4096),),
        plan=(NVFP4,), x_dist="student_t_cols", sr_seeds=tuple(range(10)))
    return w


WORKLOADS: Dict[str, Workload] = _make_workloads()
WORKLOAD_ORDER = ["linear512", "tinyllama1b", "llama7b", "llama70b", "down7b_sweep"]


def _rng(wid: int, layer_idx: int, role: int, extra: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, layer_idx, role, extra])))


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy array -> bf16 torch CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def gen_x(wl: Workload, layer_idx: int, rows: Optional[int] = None) -> torch.Tensor:
    """Activations X [T, d_in] in bf16."""
    layer = wl.layers[layer_idx]
    T = wl.tokens if rows is None else rows
    rng = _rng(wl.wid, layer_idx, ROLE_X)
    x = rng.standard_normal((T, layer.d_in), dtype=np.float32)
    if wl.x_dist == "normal_outliers":
        n = x.size
        k = max(1, n // 1000)           # 0.1 % of the entries
        idx = rng.choice(n, size=k, replace=False)
        x.reshape(-1)[idx] *= 20.0
    elif wl.x_dist == "student_t_cols":
        ncol = max(1, layer.d_in // 100)  # 1 % of the input channels
        cols = np.sort(rng.choice(layer.d_in, size=ncol, replace=False))
        x[:, cols] = rng.standard_t(3.0, size=(T, ncol)).astype(np.float32)
    return to_bf16(x)


def gen_w(wl: Workload, layer_idx: int) -> torch.Tensor:
    """Weights W [d_out, d_in] in bf16, N(0, w_std)."""
    layer = wl.layers[layer_idx]
    rng = _rng(wl.wid, layer_idx, ROLE_W)
    w = rng.standard_normal((layer.d_out, layer.d_in), dtype=np.float32)
    w *= np.float32(wl.w_std)
    return to_bf16(w)


def gen_dy(wl: Workload, layer_idx: int, rows: Optional[int] = None) -> torch.Tensor:
    """Upstream gradient dY [T, d_out] in bf16, N(0, dy_std)."""
    layer = wl.layers[layer_idx]
    T = wl.tokens if rows is None else rows
    rng = _rng(wl.wid, layer_idx, ROLE_DY)
    g = rng.standard_normal((T, layer.d_out), dtype=np.float32)
    g *= np.float32(wl.dy_std)
    return to_bf16(g)


def gen_layer(wl: Workload, layer_idx: int):
    return gen_x(wl, layer_idx), gen_w(wl, layer_idx), gen_dy(wl, layer_idx)


def gen_matrix(shape, seed: int, std: float = 1.0, dist: str = "normal") -> torch.Tensor:
    """Generic seeded bf16 matrix for tests that need arbitrary shapes."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([99, seed])))
    if dist == "normal":
        a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    elif dist == "uniform":
        a = (rng.random(shape, dtype=np.float32) * 2 - 1) * np.float32(std)
    elif dist == "student_t":
        a = rng.standard_t(3.0, size=shape).astype(np.float32) * np.float32(std)
    elif dist == "lognormal_mixed":
        # wide dynamic range: magnitudes spread over ~2^-20 .. 2^8
        mag = np.exp2(rng.uniform(-20, 8, size=shape)).astype(np.float32)
        sign = np.where(rng.random(shape) < 0.5, -1.0, 1.0).astype(np.float32)
        a = mag * sign * np.float32(std)
    else:
        raise ValueError(dist)
    return to_bf16(a)


def fixed_bits(seed: int, n: int) -> np.ndarray:
    """n seeded uint16 patterns (used to draw arbitrary bf16 bit patterns)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([77, seed])))
    return rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)


def bf16_from_bits(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(t: torch.Tensor) -> np.ndarray:
    """Exact bf16 -> fp32 widening as a numpy array."""
    b = bf16_bits(t).astype(np.uint32) << 16
    return b.view(np.float32)


def all_workloads() -> List[Workload]:
    return [WORKLOADS[n] for n in WORKLOAD_ORDER]
