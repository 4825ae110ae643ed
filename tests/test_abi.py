"""The C ABI on the CPU: the library loads, exports every declared entry point,
and rejects invalid arguments on the host before any GPU work is enqueued."""

import ctypes
import os
import re

import pytest

import int4_quantized_moe_amd as kt
from int4_quantized_moe_amd import _lib

from .conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kt_rawint4.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kt_rawint4_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIBRARY_PATH)
    names = _declared()
    assert len(names) == 19
    for name in names:
        assert hasattr(lib, name), name


def test_static_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define KT_RAWINT4_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m, "KT_RAWINT4_STATIC_SCRATCH_BYTES not found"
    assert _lib.KT_RAWINT4_STATIC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))


def test_profile_phase_names():
    names = [kt.kt_rawint4_profile_phase_name(i) for i in range(18)]
    assert names[0] == "group" and "scales_fp16" in names and "gemm_gate_up" in names and "h_rows" in names
    assert names[-1] == "lora_grads" and len(set(names)) == 18
    assert kt.kt_rawint4_profile_phase_name(18) == ""
    kt.kt_rawint4_profile_enable(False)
    assert sum(n for _, n in kt.kt_rawint4_profile_read().values()) == 0


def test_weight_layout(golden):
    rows = dict((r[0], r[1]) for r in golden("layout.txt"))
    assert kt.kt_rawint4_weight_layout() == rows["layout"]


FAKE = 1 << 20  # a non-null, 256-aligned address; never dereferenced by the host checks


def _layer(**over):
    args = dict(num_experts=8, top_k=2, hidden=512, intermediate=384, rank=8, alpha=16.0, swiglu_limit=2.0)
    args.update(over)
    ptrs = [over.pop(n, FAKE) for n in ("gp", "up", "dp", "gs", "us", "ds", "a0", "a1", "a2", "a3", "a4", "a5")]
    return kt.make_layer(args["num_experts"], args["top_k"], args["hidden"], args["intermediate"], args["rank"],
                         args["alpha"], args["swiglu_limit"], *ptrs)


def test_workspace_bytes_scales_with_tokens():
    small = kt.kt_rawint4_moe_workspace_bytes(_layer(), 5)
    big = kt.kt_rawint4_moe_workspace_bytes(_layer(), 500)
    assert 0 < small < big and small % 256 == 0


@pytest.mark.parametrize(
    "over, message",
    [
        (dict(num_experts=0), "num_experts"),
        (dict(top_k=9), "top_k"),
        (dict(hidden=500), "hidden"),
        (dict(intermediate=100), "intermediate"),
        (dict(rank=0), "rank"),
        (dict(rank=129), "rank"),
        (dict(swiglu_limit=-1.0), "swiglu_limit"),
        (dict(swiglu_limit=float("inf")), "swiglu_limit"),
        (dict(alpha=float("nan")), "alpha"),
    ],
)
def test_invalid_layers_are_rejected(over, message):
    layer = _layer(**over)
    with pytest.raises(kt.KtRawInt4Error, match=message) as err:
        kt.kt_rawint4_moe_workspace_bytes(layer, 4)
    assert err.value.code == kt.KT_RAWINT4_EINVAL
    lib = _lib.load_library()
    assert lib.kt_rawint4_moe_fwd(ctypes.byref(layer), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert message in kt.kt_rawint4_last_error()


def test_null_weight_pointer_rejected():
    lib = _lib.load_library()
    layer = _layer()
    layer.down_scale = None
    assert lib.kt_rawint4_moe_fwd(ctypes.byref(layer), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert "NULL" in kt.kt_rawint4_last_error()


def test_misaligned_and_small_workspace_rejected():
    lib = _lib.load_library()
    layer = _layer()
    need = kt.kt_rawint4_moe_workspace_bytes(layer, 4)
    rc = lib.kt_rawint4_moe_fwd(ctypes.byref(layer), 4, FAKE, FAKE, FAKE, FAKE, FAKE, need - 256, None)
    assert rc == kt.KT_RAWINT4_EWORKSPACE
    rc = lib.kt_rawint4_moe_fwd(ctypes.byref(layer), 4, FAKE, FAKE, FAKE, FAKE, FAKE + 8, need, None)
    assert rc == kt.KT_RAWINT4_EINVAL and "aligned" in kt.kt_rawint4_last_error()
    rc = lib.kt_rawint4_moe_fwd(ctypes.byref(layer), -1, FAKE, FAKE, FAKE, FAKE, FAKE, need, None)
    assert rc == kt.KT_RAWINT4_EINVAL and "qlen" in kt.kt_rawint4_last_error()
    layer.gate_packed = FAKE + 4
    rc = lib.kt_rawint4_moe_fwd(ctypes.byref(layer), 4, FAKE, FAKE, FAKE, FAKE, FAKE, need, None)
    assert rc == kt.KT_RAWINT4_EINVAL and "16-byte" in kt.kt_rawint4_last_error()


def test_backward_argument_checks():
    lib = _lib.load_library()
    layer = _layer()
    need = kt.kt_rawint4_moe_workspace_bytes(layer, 4)
    grads = [FAKE] * 6
    base = [ctypes.byref(layer), 4, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    rc = lib.kt_rawint4_moe_bwd(*base, *grads[:5], None, 0, 1.0, FAKE, need, None)
    assert rc == kt.KT_RAWINT4_EINVAL and "gradient" in kt.kt_rawint4_last_error()
    rc = lib.kt_rawint4_moe_bwd(*base, *grads, 0, float("nan"), FAKE, need, None)
    assert rc == kt.KT_RAWINT4_EINVAL and "grad_scale" in kt.kt_rawint4_last_error()
    rc = lib.kt_rawint4_moe_bwd(*base, *grads, 0, 1.0, FAKE, 64, None)
    assert rc == kt.KT_RAWINT4_EWORKSPACE


def test_hook_argument_checks():
    lib = _lib.load_library()
    assert lib.kt_rawint4_unpack(FAKE, 4, 3, FAKE, None) == kt.KT_RAWINT4_EINVAL
    assert lib.kt_rawint4_dequant(FAKE, FAKE, 4, 48, FAKE, None) == kt.KT_RAWINT4_EINVAL
    assert lib.kt_rawint4_group(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, 1 << 20, None) == kt.KT_RAWINT4_EINVAL
    need = kt.kt_rawint4_group_workspace_bytes(4, 2, 8)
    assert lib.kt_rawint4_group(FAKE, 4, 2, 8, FAKE, FAKE, FAKE, need - 1, None) == kt.KT_RAWINT4_EWORKSPACE
    assert lib.kt_rawint4_moe_diagnostics(None, 0, None, None, None) == kt.KT_RAWINT4_EINVAL


def test_inference_workspace_and_base_only_layer():
    layer = _layer()
    train = kt.kt_rawint4_moe_workspace_bytes(layer, 500)
    infer = kt.kt_rawint4_moe_infer_workspace_bytes(layer, 500)
    assert 0 < infer < train and infer % 256 == 0
    base = _layer(**{n: None for n in ("a0", "a1", "a2", "a3", "a4", "a5")}, rank=0, alpha=float("nan"))
    # all six LoRA pointers NULL: only the inference forward accepts it, and rank/alpha are not used
    assert 0 < kt.kt_rawint4_moe_infer_workspace_bytes(base, 500) < infer
    with pytest.raises(kt.KtRawInt4Error, match="rank"):
        kt.kt_rawint4_moe_workspace_bytes(base, 500)
    partial = _layer(a3=None)
    with pytest.raises(kt.KtRawInt4Error, match="NULL"):
        kt.kt_rawint4_moe_infer_workspace_bytes(partial, 500)
    lib = _lib.load_library()
    need = kt.kt_rawint4_moe_infer_workspace_bytes(base, 4)
    assert lib.kt_rawint4_moe_infer(ctypes.byref(base), 4, FAKE, FAKE, FAKE, FAKE, FAKE, need - 256, None) == \
        kt.KT_RAWINT4_EWORKSPACE
    assert lib.kt_rawint4_moe_infer(ctypes.byref(base), 4, None, FAKE, FAKE, FAKE, FAKE, need, None) == \
        kt.KT_RAWINT4_EINVAL
    assert lib.kt_rawint4_moe_infer(ctypes.byref(base), 0, None, None, None, None, None, 0, None) == kt.KT_RAWINT4_OK


def test_weight_format_is_validated():
    layer = _layer()
    assert layer.weight_format == kt.KT_RAWINT4_FORMAT_RAWINT4
    mx = _layer()
    mx.weight_format = kt.KT_RAWINT4_FORMAT_MXFP4
    assert kt.kt_rawint4_moe_workspace_bytes(mx, 7) == kt.kt_rawint4_moe_workspace_bytes(layer, 7)
    bad = _layer()
    bad.weight_format = 2
    with pytest.raises(kt.KtRawInt4Error, match="weight_format"):
        kt.kt_rawint4_moe_workspace_bytes(bad, 7)
    lib = _lib.load_library()
    assert lib.kt_rawint4_moe_infer(ctypes.byref(bad), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert "weight_format" in kt.kt_rawint4_last_error()
    assert lib.kt_rawint4_dequant_mxfp4(FAKE, FAKE, 4, 48, FAKE, None) == kt.KT_RAWINT4_EINVAL
    named = kt.make_layer(8, 2, 512, 384, 8, 16.0, 2.0, *([FAKE] * 12), weight_format="mxfp4")
    assert named.weight_format == kt.KT_RAWINT4_FORMAT_MXFP4
