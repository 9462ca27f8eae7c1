"""Seeded synthetic inputs for split-KV grouped-query decode attention.

This module only draws numbers; it holds none of the attention arithmetic. Both
sides use it: the HIP path (through tests and the benchmark) and the fp64
oracle. No value here is ever produced by either of them.

Seeds: ``numpy.random.default_rng([cfg_id, layer, stream_id, ...])`` with
stream 0 = q, 1 = K, 2 = V, 3 = per-block score offsets, 4 = sequence lengths.
q is fp32 N(0, 1); K and V are fp32 N(0, 1) rounded to fp16 (round to nearest
even, numpy ``astype``). Cache layout: ``[batch][max_ctx][n_kv_head][head_dim]``
(row of position p, KV head g at ``(p * n_kv_head + g) * head_dim``).

Workloads (all synthetic; the pages name no dataset):
  1 tiny      1 layer, B=1, 4q/2kv, hd 64, nkv 256, 4 splits
  2 7b_2k     28 layers, B=1, 28q/4kv, hd 128, nkv 2048 (the 7B decode shape at
              2K context of "10 · R4 — decode split-attention dim-parallel
              rewrite", section 1)
  3 growing   28q/4kv hd 128, max_ctx 33024; live lengths 2^k-1, 2^k, 2^k+1 for
              k = 7..15; K rows carry per-128-position score offsets drawn from
              U[-20, 20] so that split maxima differ widely
  4 hd256     12 layers, B=1, 16q/2kv, hd 256, nkv 8400 (the shape and context of
              "Red Lite dev35 — long-context decode: grouped split-K attention",
              Finding and Scope boundary)
  5 ragged    B=32, 32q/8kv, hd 128, max_ctx 32768, nkv_b ~ U{512..32768}
  5p          precision stress: B=1, 4q/2kv, hd 8 and 16, nkv 1024
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

F16_NAN_BITS = np.uint16(0x7E00)


@dataclass(frozen=True)
class Shape:
    batch: int
    n_head: int
    n_kv_head: int
    head_dim: int
    max_ctx: int

    @property
    def group(self) -> int:
        return self.n_head // self.n_kv_head

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))


@dataclass
class Case:
    shape: Shape
    q: np.ndarray            # fp32 [B][nh][hd]
    k: np.ndarray            # fp16 [B][max_ctx][nkvh][hd]
    v: np.ndarray            # fp16 [B][max_ctx][nkvh][hd]
    positions: np.ndarray    # int32 [B]; live length = positions[b] + 1
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def nkv(self) -> np.ndarray:
        return np.clip(self.positions.astype(np.int64) + 1, 0,
                       self.shape.max_ctx)


# Workload shapes ---------------------------------------------------------
CFG1 = Shape(1, 4, 2, 64, 256)
CFG2 = Shape(1, 28, 4, 128, 2048)
CFG3 = Shape(1, 28, 4, 128, 33024)
CFG4 = Shape(1, 16, 2, 256, 8400)
CFG5 = Shape(32, 32, 8, 128, 32768)
CFG5P = {8: Shape(1, 4, 2, 8, 1024), 16: Shape(1, 4, 2, 16, 1024)}

CFG1_SPLITS = 4
CFG2_LAYERS = 28
CFG2_SPLIT_SWEEP = (4, 8, 16, 32, 64)
CFG3_LAYERS = 28
CFG3_LENGTHS = tuple(n for k in range(7, 16) for n in (2**k - 1, 2**k, 2**k + 1))
CFG4_LAYERS = 12
CFG4_NKV = 8400
CFG4_BLOCKS = (32, 64, 128, 256)
CFG5_RANGE = (512, 32768)
CFG5P_NKV = 1024
OFFSET_BLOCK = 128
OFFSET_RANGE = 20.0


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(x) for x in key])


def _normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_q(cfg_id, layer, shape: Shape) -> np.ndarray:
    return _rng(cfg_id, layer, 0).standard_normal(
        (shape.batch, shape.n_head, shape.head_dim), dtype=np.float32)


def make_cache(cfg_id, layer, shape: Shape, stream: int, live=None,
               poison_tail: bool = False) -> np.ndarray:
    """fp16 [B][max_ctx][nkvh][hd]; sequence b is drawn from its own seed.

    Rows at or past ``live[b]`` are zero, or fp16 NaN with ``poison_tail`` (a
    kernel that reads past the live length then produces NaN).
    """
    B, T, H, D = shape.batch, shape.max_ctx, shape.n_kv_head, shape.head_dim
    out = np.empty((B, T, H, D), np.float16)
    live = [T] * B if live is None else [int(min(max(n, 0), T)) for n in live]

    def fill(b):
        n = live[b]
        out[b, :n] = _normal_f16(_rng(cfg_id, layer, stream, b), (n, H, D))
        tail = out[b, n:].view(np.uint16)
        tail[...] = F16_NAN_BITS if poison_tail else 0

    if B * T * H * D > (1 << 24) and B > 1:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(B)))
    else:
        for b in range(B):
            fill(b)
    return out


def make_case(cfg_id, shape: Shape, nkv, layer: int = 0,
              poison_tail: bool = False) -> Case:
    """Plain N(0,1) case with live lengths ``nkv`` (int or one per sequence)."""
    nkv = np.broadcast_to(np.asarray(nkv, np.int64), (shape.batch,))
    positions = (nkv - 1).astype(np.int32)
    q = make_q(cfg_id, layer, shape)
    k = make_cache(cfg_id, layer, shape, 1, nkv, poison_tail)
    v = make_cache(cfg_id, layer, shape, 2, nkv, poison_tail)
    return Case(shape, q, k, v, positions, shape.scale,
                {"cfg": cfg_id, "layer": layer})


def offset_direction(q_group: np.ndarray, scale: float) -> np.ndarray:
    """u with scale * (q_g . u) = 1 for every query head g of one KV group.

    u = Q^T (Q Q^T)^{-1} 1 / scale, in double (Q: G x hd, rows independent).
    Adding delta * u to a K row raises that row's score by delta for the
    whole group.
    """
    Q = q_group.astype(np.float64)
    G = Q.shape[0]
    return Q.T @ np.linalg.solve(Q @ Q.T, np.ones(G)) / float(scale)


def make_offset_case(cfg_id, shape: Shape, nkv, layer: int = 0,
                     poison_tail: bool = False) -> Case:
    """Case whose K rows carry per-128-position score offsets in [-20, 20]."""
    case = make_case(cfg_id, shape, nkv, layer, poison_tail)
    G = shape.group
    n_blocks = -(-shape.max_ctx // OFFSET_BLOCK)
    deltas = _rng(cfg_id, layer, 3).uniform(-OFFSET_RANGE, OFFSET_RANGE,
                                            (shape.batch, n_blocks))
    for b in range(shape.batch):
        n = int(case.nkv[b])
        if n == 0:
            continue
        delta_row = np.repeat(deltas[b], OFFSET_BLOCK)[:n]          # [n]
        for g in range(shape.n_kv_head):
            u = offset_direction(case.q[b, g * G:(g + 1) * G], case.scale)
            base = _rng(cfg_id, layer, 1, b, 1000 + g).standard_normal(
                (n, shape.head_dim), dtype=np.float32).astype(np.float64)
            case.k[b, :n, g, :] = (base + delta_row[:, None] * u[None, :]
                                   ).astype(np.float16)
    case.meta["offsets"] = True
    return case


def cfg5_lengths(batch: int = CFG5.batch) -> np.ndarray:
    lo, hi = CFG5_RANGE
    return _rng(5, 0, 4).integers(lo, hi, size=batch, endpoint=True)


def kv_bytes(n_kv_head: int, head_dim: int, nkv) -> int:
    """Algorithmic K+V bytes of one layer: 2 (K and V) * rows * heads * hd * 2 B."""
    return int(2 * int(np.sum(nkv)) * n_kv_head * head_dim * 2)
