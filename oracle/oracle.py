"""Python face of the CPU oracle (test infrastructure only).

The arithmetic lives in ``rawint4_oracle.c`` (fp64 accumulation); this module
marshals numpy arrays into it and adds the pages' metric and storage hash.
Sources, all on the page "rawint4_sft_reference.py":

* ``relative_l2_and_cosine``: relative L2 = |a - e| / max(|e|, 1e-12) and
  cosine = <a, e> / max(|a| |e|, 1e-20);
* ``tensor_storage_hash`` / ``base_storage_hash``: SHA-256 over the raw bytes of
  each tensor, each preceded by its byte length as 8 little-endian bytes, the
  projections taken per expert in gate, up, down order, packed codes before
  scales;
* ``finalize_window``: the optimizer-window rule of the contract test
  ("test_rawint4_sft_numerical.py", ``_expected_window`` and the lazy clear):
  a call with accumulate = False overwrites every expert row, a call with
  accumulate = True adds; each call contributes grad_scale times its gradient.
"""

from __future__ import annotations

import ctypes
import hashlib
import os
from typing import Dict, Iterable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

LORA_NAMES = ("gate_lora_a", "gate_lora_b", "up_lora_a", "up_lora_b", "down_lora_a", "down_lora_b")

# weight formats: signed group-32 RAWINT4, or MXFP4 (E2M1 nibbles, power-of-two
# UE8M0 group scales handed over as bf16)
FORMATS = {"rawint4": 0, "mxfp4": 1}

_u8p = ctypes.POINTER(ctypes.c_uint8)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


class OrcLayer(ctypes.Structure):
    _fields_ = [
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("fp32_intermediates", ctypes.c_int32),
        ("weight_format", ctypes.c_int32),
        ("alpha", ctypes.c_double),
        ("swiglu_limit", ctypes.c_double),
        ("gate_packed", _u8p),
        ("up_packed", _u8p),
        ("down_packed", _u8p),
        ("gate_scale", _u16p),
        ("up_scale", _u16p),
        ("down_scale", _u16p),
        ("gate_a", _f64p),
        ("gate_b", _f64p),
        ("up_a", _f64p),
        ("up_b", _f64p),
        ("down_a", _f64p),
        ("down_b", _f64p),
    ]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_unpack.argtypes = [_u8p, ctypes.c_int64, _i8p]
    lib.orc_pack.argtypes = [_i32p, ctypes.c_int64, _u8p]
    lib.orc_pack.restype = ctypes.c_int
    lib.orc_validate_layout.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int32]
    lib.orc_validate_layout.restype = ctypes.c_int
    lib.orc_dequant.argtypes = [_u8p, _u16p, ctypes.c_int64, ctypes.c_int64, _f32p]
    lib.orc_dequant.restype = ctypes.c_int
    lib.orc_dequant_format.argtypes = [_u8p, _u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _f32p]
    lib.orc_dequant_format.restype = ctypes.c_int
    lib.orc_e2m1_table.argtypes = [_f64p]
    lib.orc_transpose_free_dx.argtypes = [_f64p, ctypes.c_int64, _u8p, _u16p, ctypes.c_int64, ctypes.c_int64, _f64p]
    lib.orc_transpose_free_dx.restype = ctypes.c_int
    lib.orc_transpose_free_dx_format.argtypes = [_f64p, ctypes.c_int64, _u8p, _u16p, ctypes.c_int64,
                                                 ctypes.c_int64, ctypes.c_int32, _f64p]
    lib.orc_transpose_free_dx_format.restype = ctypes.c_int
    lib.orc_group.argtypes = [_i64p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _i32p, _i32p, _i32p, _i64p]
    lib.orc_group.restype = ctypes.c_int
    lib.orc_moe.argtypes = [ctypes.POINTER(OrcLayer), ctypes.c_int64, _f64p, _i64p, _f64p, _f64p, _f64p, _f64p,
                            _f64p] + [_f64p] * 6
    lib.orc_moe.restype = ctypes.c_int
    lib.orc_moe_decided.argtypes = lib.orc_moe.argtypes + [_f64p, _f64p, ctypes.c_double, _f64p, _f64p, _f64p,
                                                           _f64p]
    lib.orc_moe_decided.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray], ptype):
    if a is None:
        return ctypes.cast(None, ptype)
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ptype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


# ----------------------------------------------------------------- codec


def unpack(packed: np.ndarray) -> np.ndarray:
    """Signed values c - 8, low nibble first; shape [..., 2 * last]."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    _load().orc_unpack(_ptr(p, _u8p), p.size, _ptr(out, _i8p))
    return out


def pack(codes: np.ndarray) -> np.ndarray:
    """Pack integer codes in [0, 15]; raises ValueError like the pages' packer."""
    c = np.ascontiguousarray(codes, dtype=np.int32)
    if c.ndim < 1 or c.shape[-1] % 2:
        raise ValueError("RAWINT4 code count must be even")
    out = np.empty(c.shape[:-1] + (c.shape[-1] // 2,), dtype=np.uint8)
    rc = _load().orc_pack(_ptr(c, _i32p), c.size, _ptr(out, _u8p))
    if rc == -2:
        raise ValueError("RAWINT4 codes must be in [0, 15]")
    if rc != 0:
        raise ValueError("RAWINT4 code count must be even")
    return out


def validate_layout(packed: np.ndarray, scales: np.ndarray, group_size: int = 32):
    if packed.dtype != np.uint8 or packed.ndim != 2:
        raise ValueError("packed RAWINT4 weights must be a rank-2 uint8 array")
    if scales.dtype != np.uint16 or scales.ndim != 2:
        raise ValueError("RAWINT4 scales must be a rank-2 bf16 (uint16 bits) array")
    rc = _load().orc_validate_layout(packed.shape[0], packed.shape[1], scales.shape[0], scales.shape[1], group_size)
    if rc == -1:
        raise ValueError(f"RAWINT4 requires group_size=32, got {group_size}")
    if rc == -2:
        raise ValueError("RAWINT4 K must be divisible by group_size")
    if rc == -3:
        raise ValueError("RAWINT4 scales must have shape [N, K/32]")
    return packed.shape[0], packed.shape[1] * 2


def e2m1_table() -> np.ndarray:
    """Value of each E2M1 nibble 0..15 (unscaled)."""
    out = np.empty(16)
    _load().orc_e2m1_table(_ptr(out, _f64p))
    return out


def dequant(packed: np.ndarray, scales: np.ndarray, weight_format: str = "rawint4") -> np.ndarray:
    n, k = validate_layout(packed, scales)
    out = np.empty((n, k), dtype=np.float32)
    rc = _load().orc_dequant_format(_ptr(np.ascontiguousarray(packed), _u8p), _ptr(np.ascontiguousarray(scales), _u16p),
                                    n, k, FORMATS[weight_format], _ptr(out, _f32p))
    assert rc == 0
    return out


def transpose_free_dx(dy: np.ndarray, packed: np.ndarray, scales: np.ndarray, weight_format: str = "rawint4") -> np.ndarray:
    n, k = validate_layout(packed, scales)
    d = np.ascontiguousarray(dy, dtype=np.float64)
    if d.ndim != 2 or d.shape[1] != n:
        raise ValueError(f"grad_output must have shape [M, {n}]")
    out = np.empty((d.shape[0], k), dtype=np.float64)
    rc = _load().orc_transpose_free_dx_format(_ptr(d, _f64p), d.shape[0], _ptr(np.ascontiguousarray(packed), _u8p),
                                              _ptr(np.ascontiguousarray(scales), _u16p), n, k,
                                              FORMATS[weight_format], _ptr(out, _f64p))
    assert rc == 0
    return out


def group(expert_ids: np.ndarray, num_experts: int):
    """(counts[E], offsets[E+1], sorted_slot[valid], bad) by stable counting sort."""
    ids = np.ascontiguousarray(expert_ids, dtype=np.int64)
    qlen, top_k = ids.shape
    counts = np.empty(num_experts, dtype=np.int32)
    offsets = np.empty(num_experts + 1, dtype=np.int32)
    sorted_slot = np.full(ids.size, -1, dtype=np.int32)
    bad = ctypes.c_int64(0)
    rc = _load().orc_group(_ptr(ids, _i64p), qlen, top_k, num_experts, _ptr(counts, _i32p), _ptr(offsets, _i32p),
                           _ptr(sorted_slot, _i32p), ctypes.byref(bad))
    if rc:
        raise ValueError("invalid grouping arguments")
    return counts, offsets, sorted_slot[: int(offsets[-1])], int(bad.value)


# ----------------------------------------------------------------- layer


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


APRIORI = -1.0  # band: each element's a priori fp32 error bound (see the oracle's preact_bound)


def moe(cfg, weights, inputs, expert_ids, route_weights, grad_output=None, *, fp32_intermediates=True,
        inputs_are_bf16=True, lora: Optional[Dict[str, np.ndarray]] = None, sides=None, band=0.0,
        preactivations=False):
    """Forward (and, with ``grad_output``, backward) of the routed layer.

    ``inputs`` / ``grad_output`` are bf16 bit patterns when ``inputs_are_bf16``,
    else float arrays used as given.  Returns a dict with ``out`` [qlen, H] and,
    for the backward, ``dx``, ``droute`` [qlen, k] and the six raw LoRA
    gradients (sums over this call's tokens, before the window rule).

    ``sides = (gate, up)``, each [qlen, k, I]: pre-activations found by the
    computation under test; where the oracle's own value is within ``band`` of
    a clamp bound, its mask follows the side of the supplied value (the mask is
    not unique there).  ``band = APRIORI`` takes each element's a priori bound
    on the error of an fp32 computation of it instead.  ``preactivations`` adds
    the oracle's own ``pre_g`` / ``pre_u`` [qlen, k, I] (zero for dropped
    slots) and their a priori bounds ``bound_g`` / ``bound_u``.
    """
    lib = _load()
    lora = weights.lora if lora is None else lora
    h, i, r, e = cfg.hidden, cfg.intermediate, cfg.rank, cfg.num_experts
    keep = {name: np.ascontiguousarray(lora[name], dtype=np.float64) for name in LORA_NAMES}
    arrays = [np.ascontiguousarray(a) for a in (weights.gate_packed, weights.up_packed, weights.down_packed,
                                                 weights.gate_scale, weights.up_scale, weights.down_scale)]
    fmt = FORMATS[getattr(cfg, "weight_format", "rawint4")]
    layer = OrcLayer(e, cfg.top_k, h, i, r, 1 if fp32_intermediates else 0, fmt, float(cfg.alpha), float(cfg.swiglu_limit),
                     _ptr(arrays[0], _u8p), _ptr(arrays[1], _u8p), _ptr(arrays[2], _u8p), _ptr(arrays[3], _u16p),
                     _ptr(arrays[4], _u16p), _ptr(arrays[5], _u16p), *(_ptr(keep[n], _f64p) for n in LORA_NAMES))
    x = _bf16_to_f64(inputs) if inputs_are_bf16 else np.ascontiguousarray(inputs, dtype=np.float64)
    ids = np.ascontiguousarray(expert_ids, dtype=np.int64)
    rw = np.ascontiguousarray(route_weights, dtype=np.float64)
    qlen = x.shape[0]
    assert ids.shape == rw.shape and ids.shape[0] == qlen and x.shape[1] == h
    out = np.empty((qlen, h))
    res = {"out": out}
    dy = None
    grads = [None] * 6
    dx = droute = None
    if grad_output is not None:
        dy = _bf16_to_f64(grad_output) if inputs_are_bf16 else np.ascontiguousarray(grad_output, dtype=np.float64)
        dx = np.empty((qlen, h))
        droute = np.empty(ids.shape)
        shapes = cfg.lora_shapes()
        grads = [np.empty(shapes[n]) for n in LORA_NAMES]
    side_g = side_u = pre_g = pre_u = bnd_g = bnd_u = None
    if sides is not None:
        side_g, side_u = (np.ascontiguousarray(a, dtype=np.float64).reshape(ids.shape + (i,)) for a in sides)
    if preactivations:
        pre_g = np.zeros(ids.shape + (i,))
        pre_u = np.zeros(ids.shape + (i,))
        bnd_g = np.zeros(ids.shape + (i,))
        bnd_u = np.zeros(ids.shape + (i,))
        res["pre_g"] = pre_g
        res["pre_u"] = pre_u
        res["bound_g"] = bnd_g
        res["bound_u"] = bnd_u
    rc = lib.orc_moe_decided(ctypes.byref(layer), qlen, _ptr(x, _f64p), _ptr(ids, _i64p), _ptr(rw, _f64p),
                             _ptr(dy, _f64p), _ptr(out, _f64p), _ptr(dx, _f64p), _ptr(droute, _f64p),
                             *(_ptr(g, _f64p) for g in grads), _ptr(side_g, _f64p), _ptr(side_u, _f64p), float(band),
                             _ptr(pre_g, _f64p), _ptr(pre_u, _f64p), _ptr(bnd_g, _f64p), _ptr(bnd_u, _f64p))
    if rc:
        raise RuntimeError(f"oracle failed with code {rc}")
    if dy is not None:
        res["dx"] = dx
        res["droute"] = droute
        res["grads"] = dict(zip(LORA_NAMES, grads))
    return res


def finalize_window(previous: Optional[np.ndarray], raw: np.ndarray, accumulate: bool, grad_scale: float):
    """Gradient buffer after one call: (accumulate ? previous : 0) + grad_scale * raw."""
    base = previous if (accumulate and previous is not None) else 0.0
    return base + grad_scale * raw


# ----------------------------------------------------------------- metrics and hashes


def relative_l2_and_cosine(actual, expected):
    a = np.asarray(actual, dtype=np.float64).ravel()
    e = np.asarray(expected, dtype=np.float64).ravel()
    diff = np.linalg.norm(a - e)
    en = np.linalg.norm(e)
    an = np.linalg.norm(a)
    return float(diff / max(en, 1e-12)), float(np.dot(a, e) / max(an * en, 1e-20))


def tensor_storage_hash(arrays: Iterable[np.ndarray]) -> str:
    digest = hashlib.sha256()
    for a in arrays:
        raw = np.ascontiguousarray(a).tobytes()
        digest.update(len(raw).to_bytes(8, byteorder="little"))
        digest.update(raw)
    return digest.hexdigest()


def base_storage_hash(weights) -> str:
    arrays = []
    for ex in range(weights.gate_packed.shape[0]):
        for packed, scale in ((weights.gate_packed, weights.gate_scale), (weights.up_packed, weights.up_scale),
                              (weights.down_packed, weights.down_scale)):
            arrays.extend((packed[ex], scale[ex]))
    return tensor_storage_hash(arrays)
