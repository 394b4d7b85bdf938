"""Seeded synthetic workloads with the shapes and outlier structure of the
pages' experiments.

This module only draws random inputs; it holds none of the method's
arithmetic, so both the GPU path and the CPU oracle can consume it.

Structure reproduced (OSC abstract: outliers are token-persistent, i.e. the
same few input channels are large for every token):

* ``W ~ N(0, 0.02^2)`` float32, laid out ``[K][N]`` (input channel major).
* ``X ~ N(0, 1)`` float32 ``[M][K]``; a fixed, seed-drawn set ``S`` of input
  channels is multiplied by a per-channel factor (x50 for the tiny case,
  log-uniform in [30, 100] otherwise) in both the calibration draw and the
  evaluation draw.
* Calibration draws use the same channel set and factors as the evaluation
  tokens, but independent values.

Streams: ``SeedSequence([seed, layer]).spawn(6)`` gives, in order, the
outlier-channel draw, the per-channel factors, W, X_cal, X_eval and routing.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass
class Layer:
    name: str
    m: int
    k: int
    n: int
    k_out: int
    x: np.ndarray  # [m][k] float32 evaluation tokens
    x_cal: np.ndarray  # [m_cal][k] float32 calibration tokens
    w: np.ndarray  # [k][n] float32
    scaled: np.ndarray  # sorted indices of the scaled channels
    x_dtype: str = "bf16"
    meta: dict = field(default_factory=dict)


def _streams(seed: int, layer: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence([seed, layer]).spawn(6)]


def draw_layer(name, seed, layer, m, k, n, m_cal, n_scaled, factor="loguniform", k_out=None,
               x_dtype="bf16", w_std=0.02, draw_x=True):
    r_ch, r_fac, r_w, r_cal, r_x, _ = _streams(seed, layer)
    scaled = np.sort(r_ch.choice(k, size=n_scaled, replace=False)).astype(np.int64)
    if factor == "loguniform":
        fac = np.exp(r_fac.uniform(math.log(30.0), math.log(100.0), size=n_scaled)).astype(np.float32)
    else:
        fac = np.full(n_scaled, float(factor), dtype=np.float32)
    w = r_w.standard_normal((k, n), dtype=np.float32)
    w *= np.float32(w_std)
    x_cal = r_cal.standard_normal((m_cal, k), dtype=np.float32)
    x_cal[:, scaled] *= fac
    if draw_x:
        x = r_x.standard_normal((m, k), dtype=np.float32)
        x[:, scaled] *= fac
    else:
        x = np.zeros((0, k), np.float32)
    return Layer(name=name, m=m, k=k, n=n, k_out=n_scaled if k_out is None else k_out, x=x,
                 x_cal=x_cal, w=w, scaled=scaled, x_dtype=x_dtype,
                 meta=dict(seed=seed, layer=layer, factors=fac))


# ------------------------------------------------------------------ configs
TINY = dict(m=64, k=256, n=256, m_cal=128, n_scaled=16, factor=50.0, x_dtype="f32")
LLAMA3_8B_SHAPES = [("o_proj", 4096, 4096), ("gate_up", 4096, 14336), ("down", 14336, 4096)]
LLAMA3_70B_SHAPES = [("qkvo", 8192, 8192), ("gate_up", 8192, 28672), ("down", 28672, 8192)]
FRACTIONS = {"1/2": 2, "1/4": 4, "1/8": 8, "1/16": 16}


def tiny(seed: int = 1000) -> Layer:
    c = TINY
    return draw_layer("tiny", seed, 0, c["m"], c["k"], c["n"], c["m_cal"], c["n_scaled"],
                      factor=c["factor"], x_dtype="f32")


def llama3_8b(layer: int, seed: int = 1001, m: int = 2048, m_cal: int = 512) -> Layer:
    nm, k, n = LLAMA3_8B_SHAPES[layer]
    return draw_layer("llama3_8b." + nm, seed, layer, m, k, n, m_cal, k // 16)


def llama3_70b(layer: int, frac_den: int = 16, seed: int = 1002, m: int = 4096, m_cal: int = 512,
               draw_x: bool = True) -> Layer:
    """Scaled channels are always K/16; the selected outlier count is K/frac_den."""
    nm, k, n = LLAMA3_70B_SHAPES[layer]
    return draw_layer("llama3_70b." + nm, seed, layer, m, k, n, m_cal, k // 16, k_out=k // frac_den,
                      draw_x=draw_x)


def sq_weight(seed: int = 1004, m: int = 2048, k: int = 4096, n: int = 14336, m_cal: int = 512):
    lay = draw_layer("sq_weight", seed, 0, m, k, n, m_cal, k // 16)
    lay.meta["nnz_frac"] = 8  # top 1/8 of the low weight slots per output row
    return lay


@dataclass
class MoE:
    experts: int
    tokens: int
    topk: int
    hidden: int
    inter: int
    offsets: np.ndarray  # [E+1] int64 row offsets of each expert's group
    token_of_row: np.ndarray  # [rows] token index of each grouped row
    up: list  # per-expert Layer (x = grouped rows of the hidden states)
    down: list  # per-expert Layer (fresh inputs of width inter)


def qwen3_moe(seed: int = 1003, experts: int = 128, tokens: int = 8192, topk: int = 8,
              hidden: int = 2048, inter: int = 768, cal_rows: int = 128) -> MoE:
    """Grouped expert GEMMs: tokens routed to ``topk`` distinct experts drawn
    uniformly; rows grouped by expert (ascending token order inside a group)."""
    base = _streams(seed, 0)
    r_ch, r_fac, _, _, r_x, r_route = base
    # hidden states shared by all experts' up projections
    scaled = np.sort(r_ch.choice(hidden, size=hidden // 16, replace=False)).astype(np.int64)
    fac = np.exp(r_fac.uniform(math.log(30.0), math.log(100.0), size=len(scaled))).astype(np.float32)
    h = r_x.standard_normal((tokens, hidden), dtype=np.float32)
    h[:, scaled] *= fac
    choice = np.argsort(r_route.random((tokens, experts)), axis=1)[:, :topk]
    rows_of = [np.nonzero((choice == e).any(axis=1))[0] for e in range(experts)]
    offsets = np.zeros(experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum([len(r) for r in rows_of])
    token_of_row = np.concatenate(rows_of).astype(np.int64)
    up, down = [], []
    for e in range(experts):
        _, _, r_w, r_cal, r_xd, _ = _streams(seed, 1 + e)
        w_up = r_w.standard_normal((hidden, inter), dtype=np.float32) * np.float32(0.02)
        x_cal = r_cal.standard_normal((cal_rows, hidden), dtype=np.float32)
        x_cal[:, scaled] *= fac
        up.append(Layer(name=f"moe.up.{e}", m=len(rows_of[e]), k=hidden, n=inter,
                        k_out=hidden // 16, x=h[rows_of[e]], x_cal=x_cal, w=w_up, scaled=scaled))
        dn = draw_layer(f"moe.down.{e}", seed, 1000 + e, len(rows_of[e]), inter, hidden, cal_rows,
                        inter // 16)
        down.append(dn)
    return MoE(experts, tokens, topk, hidden, inter, offsets, token_of_row, up, down)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round an fp32 input once to bf16 (the stored input format), as uint16."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)
