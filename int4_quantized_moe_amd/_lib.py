"""ctypes binding of ``libkt_rawint4.so`` (argument marshalling only).

Every function has the name and argument order of its C entry point in
``include/kt_rawint4.h``.  Tensors are passed as raw pointers (``data_ptr()``),
``stream`` defaults to torch's current HIP stream, and a nonzero return code
raises ``KtRawInt4Error`` with the library's message.  There is no fallback:
without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libkt_rawint4.so")

KT_RAWINT4_OK = 0
KT_RAWINT4_EINVAL = -1
KT_RAWINT4_EWORKSPACE = -2
KT_RAWINT4_EHIP = -3

KT_RAWINT4_STATIC_SCRATCH_BYTES = 64 << 20

KT_RAWINT4_FORMAT_RAWINT4 = 0
KT_RAWINT4_FORMAT_MXFP4 = 1
FORMATS = {"rawint4": KT_RAWINT4_FORMAT_RAWINT4, "mxfp4": KT_RAWINT4_FORMAT_MXFP4}

_vp = ctypes.c_void_p


class KtRawInt4Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"kt_rawint4 error {code}: {message}")
        self.code = code


class kt_rawint4_moe_layer(ctypes.Structure):  # noqa: N801 - the C struct's name
    _fields_ = [
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("swiglu_limit", ctypes.c_float),
        ("gate_packed", _vp),
        ("up_packed", _vp),
        ("down_packed", _vp),
        ("gate_scale", _vp),
        ("up_scale", _vp),
        ("down_scale", _vp),
        ("gate_lora_a", _vp),
        ("gate_lora_b", _vp),
        ("up_lora_a", _vp),
        ("up_lora_b", _vp),
        ("down_lora_a", _vp),
        ("down_lora_b", _vp),
        ("weight_format", ctypes.c_int32),
    ]


_lib = None


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise KtRawInt4Error(KT_RAWINT4_EHIP, f"{LIBRARY_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIBRARY_PATH)
    lp = ctypes.POINTER(kt_rawint4_moe_layer)
    i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sigs = {
        "kt_rawint4_moe_workspace_bytes": (sz, [lp, i32]),
        "kt_rawint4_moe_fwd": (ctypes.c_int, [lp, i32, _vp, _vp, _vp, _vp, _vp, sz, _vp]),
        "kt_rawint4_moe_infer_workspace_bytes": (sz, [lp, i32]),
        "kt_rawint4_moe_infer": (ctypes.c_int, [lp, i32, _vp, _vp, _vp, _vp, _vp, sz, _vp]),
        "kt_rawint4_moe_infer_static": (ctypes.c_int, [lp, i32, _vp, _vp, _vp, _vp, _vp]),
        "kt_rawint4_moe_bwd": (ctypes.c_int, [lp, i32, _vp, _vp, _vp, _vp, _vp, _vp] + [_vp] * 6 + [i32, f32, _vp, sz, _vp]),
        "kt_rawint4_moe_bwd_recompute": (ctypes.c_int,
                                         [lp, i32, _vp, _vp, _vp, _vp, _vp, _vp] + [_vp] * 6 + [i32, f32, _vp, sz, _vp]),
        "kt_rawint4_unpack": (ctypes.c_int, [_vp, i64, i64, _vp, _vp]),
        "kt_rawint4_dequant": (ctypes.c_int, [_vp, _vp, i64, i64, _vp, _vp]),
        "kt_rawint4_dequant_mxfp4": (ctypes.c_int, [_vp, _vp, i64, i64, _vp, _vp]),
        "kt_rawint4_group_workspace_bytes": (sz, [i32, i32, i32]),
        "kt_rawint4_group": (ctypes.c_int, [_vp, i32, i32, i32, _vp, _vp, _vp, sz, _vp]),
        "kt_rawint4_moe_diagnostics": (ctypes.c_int, [_vp, sz, ctypes.POINTER(i64), ctypes.POINTER(i64), _vp]),
        "kt_rawint4_moe_saved_preactivations": (ctypes.c_int, [lp, i32, _vp, sz, _vp, _vp, _vp]),
        "kt_rawint4_profile_enable": (ctypes.c_int, [i32]),
        "kt_rawint4_profile_read": (ctypes.c_int, [_vp, _vp, i32]),
        "kt_rawint4_profile_phase_name": (ctypes.c_char_p, [i32]),
        "kt_rawint4_last_error": (ctypes.c_char_p, []),
        "kt_rawint4_weight_layout": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to kt_rawint4 must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != KT_RAWINT4_OK:
        raise KtRawInt4Error(rc, kt_rawint4_last_error())


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def make_layer(num_experts, top_k, hidden, intermediate, rank, alpha, swiglu_limit, gate_packed, up_packed,
               down_packed, gate_scale, up_scale, down_scale, gate_lora_a, gate_lora_b, up_lora_a, up_lora_b,
               down_lora_a, down_lora_b, weight_format=KT_RAWINT4_FORMAT_RAWINT4) -> kt_rawint4_moe_layer:
    """Fill the C layer struct; the caller keeps the tensors alive.  weight_format:
    KT_RAWINT4_FORMAT_* or its name ("rawint4", "mxfp4")."""
    fmt = FORMATS[weight_format] if isinstance(weight_format, str) else int(weight_format)
    return kt_rawint4_moe_layer(int(num_experts), int(top_k), int(hidden), int(intermediate), int(rank), float(alpha),
                                float(swiglu_limit), _ptr(gate_packed), _ptr(up_packed), _ptr(down_packed),
                                _ptr(gate_scale), _ptr(up_scale), _ptr(down_scale), _ptr(gate_lora_a),
                                _ptr(gate_lora_b), _ptr(up_lora_a), _ptr(up_lora_b), _ptr(down_lora_a),
                                _ptr(down_lora_b), fmt)


def kt_rawint4_moe_workspace_bytes(layer: kt_rawint4_moe_layer, qlen: int) -> int:
    n = load_library().kt_rawint4_moe_workspace_bytes(ctypes.byref(layer), int(qlen))
    if n == 0:
        raise KtRawInt4Error(KT_RAWINT4_EINVAL, kt_rawint4_last_error())
    return int(n)


def kt_rawint4_moe_fwd(layer, qlen, inputs, expert_ids, route_weights, output, workspace, stream=None) -> None:
    _check(load_library().kt_rawint4_moe_fwd(ctypes.byref(layer), int(qlen), _ptr(inputs), _ptr(expert_ids),
                                             _ptr(route_weights), _ptr(output), _ptr(workspace),
                                             _nbytes(workspace) if workspace is not None else 0, _stream(stream)))


def kt_rawint4_moe_infer_workspace_bytes(layer: kt_rawint4_moe_layer, qlen: int) -> int:
    n = load_library().kt_rawint4_moe_infer_workspace_bytes(ctypes.byref(layer), int(qlen))
    if n == 0:
        raise KtRawInt4Error(KT_RAWINT4_EINVAL, kt_rawint4_last_error())
    return int(n)


def kt_rawint4_moe_infer(layer, qlen, inputs, expert_ids, route_weights, output, workspace, stream=None) -> None:
    _check(load_library().kt_rawint4_moe_infer(ctypes.byref(layer), int(qlen), _ptr(inputs), _ptr(expert_ids),
                                               _ptr(route_weights), _ptr(output), _ptr(workspace),
                                               _nbytes(workspace) if workspace is not None else 0, _stream(stream)))


def kt_rawint4_moe_infer_static(layer, qlen, inputs, expert_ids, route_weights, output, stream=None) -> None:
    _check(load_library().kt_rawint4_moe_infer_static(ctypes.byref(layer), int(qlen), _ptr(inputs), _ptr(expert_ids),
                                                      _ptr(route_weights), _ptr(output), _stream(stream)))


def kt_rawint4_moe_bwd(layer, qlen, inputs, expert_ids, route_weights, grad_output, grad_input, grad_route, d_gate_a,
                       d_gate_b, d_up_a, d_up_b, d_down_a, d_down_b, accumulate, grad_scale, workspace,
                       stream=None) -> None:
    _check(load_library().kt_rawint4_moe_bwd(
        ctypes.byref(layer), int(qlen), _ptr(inputs), _ptr(expert_ids), _ptr(route_weights), _ptr(grad_output),
        _ptr(grad_input), _ptr(grad_route), _ptr(d_gate_a), _ptr(d_gate_b), _ptr(d_up_a), _ptr(d_up_b),
        _ptr(d_down_a), _ptr(d_down_b), int(bool(accumulate)), float(grad_scale), _ptr(workspace),
        _nbytes(workspace) if workspace is not None else 0, _stream(stream)))


def kt_rawint4_moe_bwd_recompute(layer, qlen, inputs, expert_ids, route_weights, grad_output, grad_input, grad_route,
                                 d_gate_a, d_gate_b, d_up_a, d_up_b, d_down_a, d_down_b, accumulate, grad_scale,
                                 workspace, stream=None) -> None:
    _check(load_library().kt_rawint4_moe_bwd_recompute(
        ctypes.byref(layer), int(qlen), _ptr(inputs), _ptr(expert_ids), _ptr(route_weights), _ptr(grad_output),
        _ptr(grad_input), _ptr(grad_route), _ptr(d_gate_a), _ptr(d_gate_b), _ptr(d_up_a), _ptr(d_up_b),
        _ptr(d_down_a), _ptr(d_down_b), int(bool(accumulate)), float(grad_scale), _ptr(workspace),
        _nbytes(workspace) if workspace is not None else 0, _stream(stream)))


def kt_rawint4_unpack(packed, n, k, codes, stream=None) -> None:
    _check(load_library().kt_rawint4_unpack(_ptr(packed), int(n), int(k), _ptr(codes), _stream(stream)))


def kt_rawint4_dequant(packed, scales, n, k, weights, stream=None) -> None:
    _check(load_library().kt_rawint4_dequant(_ptr(packed), _ptr(scales), int(n), int(k), _ptr(weights),
                                             _stream(stream)))


def kt_rawint4_dequant_mxfp4(packed, scales, n, k, weights, stream=None) -> None:
    _check(load_library().kt_rawint4_dequant_mxfp4(_ptr(packed), _ptr(scales), int(n), int(k), _ptr(weights),
                                                   _stream(stream)))


def kt_rawint4_group_workspace_bytes(qlen, top_k, num_experts) -> int:
    n = load_library().kt_rawint4_group_workspace_bytes(int(qlen), int(top_k), int(num_experts))
    if n == 0:
        raise KtRawInt4Error(KT_RAWINT4_EINVAL, kt_rawint4_last_error())
    return int(n)


def kt_rawint4_group(expert_ids, qlen, top_k, num_experts, offsets, sorted_slot, workspace, stream=None) -> None:
    _check(load_library().kt_rawint4_group(_ptr(expert_ids), int(qlen), int(top_k), int(num_experts), _ptr(offsets),
                                           _ptr(sorted_slot), _ptr(workspace),
                                           _nbytes(workspace) if workspace is not None else 0, _stream(stream)))


def kt_rawint4_moe_diagnostics(workspace, stream=None):
    """Returns (bad_ids, bad_scales) of the latest forward; synchronises the stream."""
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(load_library().kt_rawint4_moe_diagnostics(_ptr(workspace), _nbytes(workspace), ctypes.byref(a),
                                                     ctypes.byref(b), _stream(stream)))
    return int(a.value), int(b.value)


def kt_rawint4_moe_saved_preactivations(layer, qlen, workspace, gate, up, stream=None) -> None:
    _check(load_library().kt_rawint4_moe_saved_preactivations(ctypes.byref(layer), int(qlen), _ptr(workspace),
                                                              _nbytes(workspace), _ptr(gate), _ptr(up),
                                                              _stream(stream)))


def kt_rawint4_profile_enable(on: bool) -> None:
    _check(load_library().kt_rawint4_profile_enable(1 if on else 0))


def kt_rawint4_profile_read():
    """{phase name: (milliseconds, launches)} recorded since the last read."""
    cap = 64
    ms = (ctypes.c_float * cap)()
    n = (ctypes.c_int32 * cap)()
    rc = load_library().kt_rawint4_profile_read(ctypes.addressof(ms), ctypes.addressof(n), cap)
    if rc < 0:
        raise KtRawInt4Error(rc, kt_rawint4_last_error())
    return {kt_rawint4_profile_phase_name(i): (float(ms[i]), int(n[i])) for i in range(rc)}


def kt_rawint4_profile_phase_name(phase: int) -> str:
    return load_library().kt_rawint4_profile_phase_name(int(phase)).decode()


def kt_rawint4_last_error() -> str:
    return load_library().kt_rawint4_last_error().decode()


def kt_rawint4_weight_layout() -> str:
    return load_library().kt_rawint4_weight_layout().decode()
