"""GPU: the inference forward that allocates nothing (kt_rawint4_moe_infer_static).

It runs the kernels of kt_rawint4_moe_infer in the library's own device array
instead of a caller's workspace, so its output must equal that entry point's
bit for bit (and so meet the oracle bars that kt_rawint4_moe_infer is held to:
relative L2 <= 5e-3, cosine >= 0.9999, checked here too).  Two calls in a row,
the second with fewer tokens, with LoRA and with the frozen base alone; a call
larger than the array is refused.  Each case prints its name first.
"""

import ctypes

import numpy as np
import pytest

import oracle as O
from int4_quantized_moe_amd import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[no-alloc]", *a, flush=True)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("base_only", [False, True])
def test_static_infer_equals_infer(base_only):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_quantized_moe_amd import _lib, device

    cfg, weights, batch = W.make_workload(1)  # 8 experts, top-2, hidden 512, intermediate 384, clamp 2
    dl = device.DeviceLayer(cfg, weights, base_only=base_only)
    zero = {n: np.zeros(s) for n, s in cfg.lora_shapes().items()} if base_only else None
    for qlen in (cfg.qlen, 9):  # the second call smaller than the first
        _say(f"{cfg.name}: {'base alone' if base_only else 'with LoRA'}, {qlen} tokens")
        inputs, ids, rw = batch.inputs[:qlen], batch.expert_ids[:qlen], batch.route_weights[:qlen]
        b = W.Batch(inputs=inputs, expert_ids=ids, route_weights=rw, grad_output=batch.grad_output[:qlen])
        db = device.DeviceBatch(b)
        want = dl.infer(db.inputs, db.expert_ids, db.route_weights, dl.infer_workspace(db.qlen))
        got = torch.full_like(want, float("nan"))
        _lib.kt_rawint4_moe_infer_static(dl.layer, qlen, db.inputs, db.expert_ids, db.route_weights, got)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(want)), "static-scratch output differs from kt_rawint4_moe_infer"
        ref = O.moe(cfg, weights, inputs, ids, rw, lora=zero)
        r, c = O.relative_l2_and_cosine(got.float().cpu().numpy(), ref["out"])
        _say(f"against the oracle: rel_l2={r:.3e} cos={c:.7f}")
        assert r <= 5e-3 and c >= 0.9999


def test_static_infer_refuses_a_call_beyond_its_array():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_quantized_moe_amd import _lib

    _say("a call beyond the static array")
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")  # never read: the call is refused first
    p = buf.data_ptr()
    layer = _lib.make_layer(384, 8, 7168, 2048, 16, 32.0, 0.0, *([p] * 12))
    need = _lib.load_library().kt_rawint4_moe_infer_workspace_bytes(ctypes.byref(layer), 32)
    assert need > _lib.KT_RAWINT4_STATIC_SCRATCH_BYTES
    with pytest.raises(_lib.KtRawInt4Error) as err:
        _lib.kt_rawint4_moe_infer_static(layer, 32, p, p, p, p)
    assert err.value.code == _lib.KT_RAWINT4_EWORKSPACE
