"""Seeded synthetic inputs for the RAWINT4 routed-expert LoRA layer.

This module only draws random data of the right shapes and distributions.  It
holds none of the method's arithmetic (no decode, no projection, no SwiGLU), so
both the CPU oracle and the GPU path may take their inputs from it.

Distributions follow the contract test of the pages ("test_rawint4_sft_numerical.py",
``_make_projection`` / ``_make_batch``) and the five workload configurations:

* packed codes: uniform random bytes, i.e. two independent uniform nibbles,
  low nibble first;
* group scales: fp32 uniform in [0.01, 0.07), rounded to bf16 (round to nearest even);
* MXFP4 weights (``weight_format="mxfp4"``): the same uniform bytes read as E2M1
  nibbles, and UE8M0 scale exponents uniform in [121, 124] (2^-6 .. 2^-3, so
  that the weights' magnitudes match the RAWINT4 recipe's), handed over as bf16
  by the loader's bit-cast ``e << 7``;
* activations and output gradients: N(0, 1) times a per-config std, rounded to bf16;
* LoRA A and B: fp32 N(0, 0.02);
* routing: ``top_k`` distinct experts per token, uniform or Zipf(s) over a seeded
  permutation of the experts (sampled without replacement);
* route weights: softmax over ``top_k`` N(0, 1) logits.

bf16 tensors are carried as ``uint16`` bit patterns so that numpy (which has no
bf16 type) can hold them; ``bf16_bits_to_f32`` widens them exactly.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

BASE_SEED = 20261001

LORA_NAMES = ("gate_lora_a", "gate_lora_b", "up_lora_a", "up_lora_b", "down_lora_a", "down_lora_b")


@dataclass(frozen=True)
class LayerConfig:
    name: str
    num_experts: int
    top_k: int
    hidden: int
    intermediate: int
    rank: int
    alpha: float
    qlen: int
    swiglu_limit: float
    routing: str = "uniform"  # "uniform" or "zipf"
    weight_format: str = "rawint4"  # "rawint4" or "mxfp4"
    zipf_s: float = 1.1
    x_std: float = 1.0
    dy_std: float = 1.0

    @property
    def slots(self) -> int:
        return self.qlen * self.top_k

    def lora_shapes(self) -> Dict[str, tuple]:
        e, h, i, r = self.num_experts, self.hidden, self.intermediate, self.rank
        return {
            "gate_lora_a": (e, r, h),
            "gate_lora_b": (e, i, r),
            "up_lora_a": (e, r, h),
            "up_lora_b": (e, i, r),
            "down_lora_a": (e, r, i),
            "down_lora_b": (e, h, r),
        }


# The five workloads: two small parity cases, then the Kimi-K2-like routed layer
# (384 experts, top-8, hidden 7168, intermediate 2048) at decode-like, SFT-batch
# (Zipf-skewed routing) and long-sequence (rank 64, clamp 7) token counts.
CONFIGS = (
    LayerConfig("tiny", 4, 2, 256, 256, 8, 16.0, 5, 0.0),
    LayerConfig("rect_clamp", 8, 2, 512, 384, 8, 16.0, 32, 2.0, x_std=3.0),
    LayerConfig("k2_qlen32", 384, 8, 7168, 2048, 16, 32.0, 32, 0.0),
    LayerConfig("k2_qlen4096_zipf", 384, 8, 7168, 2048, 16, 32.0, 4096, 0.0, routing="zipf"),
    LayerConfig("k2_qlen16384_r64", 384, 8, 7168, 2048, 64, 128.0, 16384, 7.0, x_std=2.0),
)


def config_seed(index: int) -> int:
    return BASE_SEED + index


def f32_to_bf16_bits(values: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 with round-to-nearest-even; returns uint16 bit patterns."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Weights:
    """Frozen RAWINT4 projections and fp32 LoRA parameters of one layer.

    ``*_packed`` are uint8 ``[E, N, K/2]`` (low nibble = even k) and ``*_scale`` are
    bf16 bits ``[E, N, K/32]``: gate/up have N = intermediate, K = hidden; down has
    N = hidden, K = intermediate.
    """

    gate_packed: np.ndarray
    up_packed: np.ndarray
    down_packed: np.ndarray
    gate_scale: np.ndarray
    up_scale: np.ndarray
    down_scale: np.ndarray
    lora: Dict[str, np.ndarray] = field(default_factory=dict)


@dataclass
class Batch:
    inputs: np.ndarray  # bf16 bits [qlen, H]
    expert_ids: np.ndarray  # int64 [qlen, top_k]
    route_weights: np.ndarray  # fp32 [qlen, top_k]
    grad_output: np.ndarray  # bf16 bits [qlen, H]


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _codes(rng: np.random.Generator, shape) -> np.ndarray:
    count = int(np.prod(shape))
    return np.frombuffer(rng.bytes(count), dtype=np.uint8).reshape(shape).copy()


def _scales(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.uniform(0.01, 0.07, size=shape).astype(np.float32))


def ue8m0_to_bf16_bits(exponents: np.ndarray) -> np.ndarray:
    """UE8M0 scale bytes to bf16 bit patterns by the loaders' bit-cast (e << 7)."""
    return (np.asarray(exponents, dtype=np.uint16) << 7).astype(np.uint16)


def _ue8m0_scales(rng: np.random.Generator, shape) -> np.ndarray:
    return ue8m0_to_bf16_bits(rng.integers(121, 125, size=shape))


def make_weights(cfg: LayerConfig, seed: int) -> Weights:
    """Draw the layer's packed codes, bf16 scales and fp32 LoRA tensors."""
    rs = _streams(seed, 12)
    e, h, i = cfg.num_experts, cfg.hidden, cfg.intermediate
    if cfg.weight_format not in ("rawint4", "mxfp4"):
        raise ValueError(f"unknown weight format {cfg.weight_format!r}")
    scales = _ue8m0_scales if cfg.weight_format == "mxfp4" else _scales
    w = Weights(
        gate_packed=_codes(rs[0], (e, i, h // 2)),
        up_packed=_codes(rs[1], (e, i, h // 2)),
        down_packed=_codes(rs[2], (e, h, i // 2)),
        gate_scale=scales(rs[3], (e, i, h // 32)),
        up_scale=scales(rs[4], (e, i, h // 32)),
        down_scale=scales(rs[5], (e, h, i // 32)),
    )
    for j, (name, shape) in enumerate(cfg.lora_shapes().items()):
        w.lora[name] = rs[6 + j].normal(0.0, 0.02, size=shape).astype(np.float32)
    return w


def _distinct_ids(rng: np.random.Generator, qlen: int, top_k: int, probs: Optional[np.ndarray], n_exp: int):
    """``top_k`` distinct experts per token; Gumbel top-k equals sampling without replacement."""
    if probs is None:
        keys = rng.random((qlen, n_exp))
    else:
        keys = np.log(probs)[None, :] + rng.gumbel(size=(qlen, n_exp))
    part = np.argpartition(-keys, top_k - 1, axis=1)[:, :top_k]
    # order each token's picks by decreasing key, the order a sequential draw would give
    order = np.argsort(-np.take_along_axis(keys, part, axis=1), axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1).astype(np.int64)


def _batch_streams(seed: int):
    return _streams(seed + 7_000_000, 5)


def _routing(cfg: LayerConfig, rs, q: int):
    probs = None
    if cfg.routing == "zipf":
        ranks = np.arange(1, cfg.num_experts + 1, dtype=np.float64)
        p_rank = ranks ** (-cfg.zipf_s)
        perm = rs[2].permutation(cfg.num_experts)
        probs = np.empty(cfg.num_experts)
        probs[perm] = p_rank / p_rank.sum()
    ids = _distinct_ids(rs[3], q, cfg.top_k, probs, cfg.num_experts)
    logits = rs[4].standard_normal((q, cfg.top_k))
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    rw = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(rw)


def make_routing(cfg: LayerConfig, seed: int, qlen: Optional[int] = None):
    """Expert ids and route weights only (identical to those of ``make_batch``)."""
    q = cfg.qlen if qlen is None else qlen
    return _routing(cfg, _batch_streams(seed), q)


def make_batch(cfg: LayerConfig, seed: int, qlen: Optional[int] = None) -> Batch:
    """Draw inputs, routing, route weights and the output gradient of one batch."""
    q = cfg.qlen if qlen is None else qlen
    rs = _batch_streams(seed)
    x = rs[0].standard_normal((q, cfg.hidden), dtype=np.float32) * np.float32(cfg.x_std)
    dy = rs[1].standard_normal((q, cfg.hidden), dtype=np.float32) * np.float32(cfg.dy_std)
    ids, rw = _routing(cfg, rs, q)
    return Batch(inputs=f32_to_bf16_bits(x), expert_ids=ids, route_weights=rw, grad_output=f32_to_bf16_bits(dy))


def make_workload(index: int, qlen: Optional[int] = None):
    """Weights and one batch of configuration ``index`` with its fixed seed."""
    cfg = CONFIGS[index]
    seed = config_seed(index)
    return cfg, make_weights(cfg, seed), make_batch(cfg, seed, qlen)
