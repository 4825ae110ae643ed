"""GPU: the inference forward (kt_rawint4_moe_infer) through the C ABI.

* With LoRA it runs the training forward's kernels on the same inputs and
  keeps nothing for a backward: its output must equal kt_rawint4_moe_fwd's bit
  for bit, in a smaller workspace.
* With all six LoRA pointers NULL it is the frozen base alone, the inference
  regression of the page "test_rawint4_sft_numerical.py": the output is held
  against the oracle with zero LoRA (relative L2 <= 5e-3 and cosine >= 0.9999,
  tighter than that page's 0.03 / 0.995), and the device copy of the base
  keeps its storage hash.  It also equals, value for value, the training
  forward of a layer whose LoRA matrices are all zero.

The forward is continuous at the clamp bounds (only the masks of the backward
jump there), so no clamp side is handed to the oracle.  Each case prints its
name first.
"""

import numpy as np
import pytest

import oracle as O
from int4_quantized_moe_amd import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
COSINE = 0.9999


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_quantized_moe_amd import device

    return device


def _say(*a):
    print("[infer]", *a, flush=True)


def _close(name, actual, expected):
    a = np.asarray(actual, dtype=np.float64)
    e = np.asarray(expected, dtype=np.float64)
    assert np.isfinite(a).all(), f"{name}: non-finite values"
    assert np.count_nonzero(e), f"{name}: reference has no signal"
    r, c = O.relative_l2_and_cosine(a, e)
    _say(f"{name}: rel_l2={r:.3e} cos={c:.7f}")
    assert r <= REL_L2 and c >= COSINE, f"{name}: rel_l2 {r:.3e} cos {c:.7f}"


def _zero_lora(cfg):
    return {n: np.zeros(s, dtype=np.float32) for n, s in cfg.lora_shapes().items()}


def _hash_device(dl):
    from int4_quantized_moe_amd.device import bf16_bits

    back = W.Weights(
        gate_packed=dl.gate_packed.cpu().numpy(), up_packed=dl.up_packed.cpu().numpy(),
        down_packed=dl.down_packed.cpu().numpy(), gate_scale=bf16_bits(dl.gate_scale),
        up_scale=bf16_bits(dl.up_scale), down_scale=bf16_bits(dl.down_scale))
    return O.base_storage_hash(back)


def _heights_case():
    # one expert with 150+ slots (tiles of several heights) and a clamp that engages
    cfg = W.LayerConfig("heights", 5, 2, 160, 224, 6, 12.0, 180, 2.5, x_std=2.0)
    weights = W.make_weights(cfg, 91)
    batch = W.make_batch(cfg, 91)
    batch.expert_ids[:150, 0] = 1
    batch.expert_ids[:150, 1] = np.where(batch.expert_ids[:150, 1] == 1, 3, batch.expert_ids[:150, 1])
    return cfg, weights, batch


def _case(which):
    if which == "heights":
        return _heights_case()
    return W.make_workload(which)


@pytest.mark.parametrize("which", [0, 1, "heights"])
def test_infer_with_lora_equals_training_forward(dev, which):
    cfg, weights, batch = _case(which)
    _say("with LoRA == training forward", cfg.name)
    dl = dev.DeviceLayer(cfg, weights)
    db = dev.DeviceBatch(batch)
    ws_train = dl.workspace(db.qlen)
    ws_inf = dl.infer_workspace(db.qlen)
    assert ws_inf.numel() < ws_train.numel()
    out_train = dl.forward(db.inputs, db.expert_ids, db.route_weights, ws_train)
    out_inf = dl.infer(db.inputs, db.expert_ids, db.route_weights, ws_inf)
    torch.cuda.synchronize()
    a = out_inf.view(torch.int16).cpu().numpy()
    b = out_train.view(torch.int16).cpu().numpy()
    assert np.array_equal(a, b), f"{cfg.name}: {np.count_nonzero(a != b)} output elements differ"


@pytest.mark.parametrize("which, rows", [(0, 0), (1, 0), ("heights", 0), ("heights", 16), ("heights", 96),
                                         ("heights", 128)])
def test_base_only_infer_against_oracle(dev, which, rows, monkeypatch):
    cfg, weights, batch = _case(which)
    _say("base only", cfg.name, "rows", rows or "default")
    if rows:
        monkeypatch.setenv("KT_RAWINT4_GEMM_ROWS", str(rows))
    else:
        monkeypatch.delenv("KT_RAWINT4_GEMM_ROWS", raising=False)
    before = O.base_storage_hash(weights)
    dl = dev.DeviceLayer(cfg, weights, base_only=True)
    db = dev.DeviceBatch(batch)
    ws = dl.infer_workspace(db.qlen)
    out = dl.infer(db.inputs, db.expert_ids, db.route_weights, ws)
    torch.cuda.synchronize()
    ref = O.moe(cfg, weights, batch.inputs, batch.expert_ids, batch.route_weights, lora=_zero_lora(cfg))
    _close(f"{cfg.name}.base", out.float().cpu().numpy(), ref["out"])
    assert _hash_device(dl) == before
    bad_ids, bad_scales = __import__("int4_quantized_moe_amd")._lib.kt_rawint4_moe_diagnostics(ws)
    assert bad_ids == 0 and bad_scales == 0

    # the same numbers as the training forward with all-zero LoRA matrices
    dz = dev.DeviceLayer(cfg, weights, lora=_zero_lora(cfg))
    wz = dz.workspace(db.qlen)
    out_z = dz.forward(db.inputs, db.expert_ids, db.route_weights, wz)
    torch.cuda.synchronize()
    assert torch.equal(out.float(), out_z.float()), f"{cfg.name}: base-only and zero-LoRA forwards differ"


def test_infer_empty_and_dropped(dev):
    cfg, weights, batch = W.make_workload(1)
    _say("base only, dropped ids and an empty call")
    batch.expert_ids[4, 0] = -1
    batch.expert_ids[11, 1] = cfg.num_experts + 2
    dl = dev.DeviceLayer(cfg, weights, base_only=True)
    db = dev.DeviceBatch(batch)
    ws = dl.infer_workspace(db.qlen)
    out = dl.infer(db.inputs, db.expert_ids, db.route_weights, ws)
    empty = torch.empty((0, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    dl.infer(db.inputs[:0], db.expert_ids[:0], db.route_weights[:0], ws, output=empty)
    torch.cuda.synchronize()
    bad_ids, _ = __import__("int4_quantized_moe_amd")._lib.kt_rawint4_moe_diagnostics(ws)
    assert bad_ids == 2
    ref = O.moe(cfg, weights, batch.inputs, batch.expert_ids, batch.route_weights, lora=_zero_lora(cfg))
    _close(f"{cfg.name}.dropped", out.float().cpu().numpy(), ref["out"])


@pytest.mark.parametrize("index", [3, 4])
def test_infer_full_size_sampled(dev, index):
    cfg = W.CONFIGS[index]
    _say(f"{cfg.name}: generating")
    cfg, weights, batch = W.make_workload(index)
    db = dev.DeviceBatch(batch)
    _say(f"{cfg.name}: inference with LoRA vs the training forward")
    dl = dev.DeviceLayer(cfg, weights)
    out_train = dl.forward(db.inputs, db.expert_ids, db.route_weights, dl.workspace(db.qlen))
    out_inf = dl.infer(db.inputs, db.expert_ids, db.route_weights, dl.infer_workspace(db.qlen))
    torch.cuda.synchronize()
    assert torch.equal(out_inf.view(torch.int16), out_train.view(torch.int16))
    del dl, out_train, out_inf
    _say(f"{cfg.name}: base only")
    db_ = dev.DeviceLayer(cfg, weights, base_only=True)
    out = db_.infer(db.inputs, db.expert_ids, db.route_weights, db_.infer_workspace(db.qlen))
    torch.cuda.synchronize()
    rng = np.random.default_rng(5151 + index)
    toks = np.unique(np.concatenate([[0, cfg.qlen - 1], rng.choice(cfg.qlen, 8, replace=False)]))
    _say(f"{cfg.name}: oracle on tokens {toks.tolist()}")
    ref = O.moe(cfg, weights, batch.inputs[toks], batch.expert_ids[toks], batch.route_weights[toks],
                lora=_zero_lora(cfg))
    _close(f"{cfg.name}.base", out.float().cpu().numpy()[toks], ref["out"])
