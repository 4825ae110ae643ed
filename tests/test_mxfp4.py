"""GPU parity of the MXFP4 weight format (weight_format = KT_RAWINT4_FORMAT_MXFP4).

The same layer with an MXFP4 base (E2M1 codes, power-of-two UE8M0 scales given
as bf16; page "ext_bindings.cpp" commit log, MXFP4_SFT_MOE): the decode is
bit-exact against the oracle, and forward, backward and the inference forward
are held to the bars of the RAWINT4 path (relative L2 <= 5e-3, cosine >=
0.9999; dRoute 3e-2) on the small workloads, on every tile height at two
ranks, and on sampled tokens and experts of the full-size long-sequence
workload.  Scales outside the MXFP4 domain that no power-of-two shift of
their group brings in (not a power of two, or negative) are counted.  Each
case prints its name first.
"""

import dataclasses

import numpy as np
import pytest

import oracle as O
from int4_quantized_moe_amd import workloads as W
from tests import fullsize as F
from tests.clamp_sides import reference

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

REL_L2 = 5e-3
COSINE = 0.9999
DROUTE_REL_L2 = 3e-2


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_quantized_moe_amd import device

    return device


def _say(*a):
    print("[mxfp4]", *a, flush=True)


def _mx(cfg):
    return dataclasses.replace(cfg, name=cfg.name + "_mxfp4", weight_format="mxfp4")


def _close(name, actual, expected, rel=REL_L2, cos=COSINE):
    a = np.asarray(actual, dtype=np.float64)
    e = np.asarray(expected, dtype=np.float64)
    assert np.isfinite(a).all(), f"{name}: non-finite values"
    assert np.count_nonzero(e), f"{name}: reference has no signal"
    r, c = O.relative_l2_and_cosine(a, e)
    _say(f"{name}: rel_l2={r:.3e} cos={c:.7f}")
    assert r <= rel and c >= cos, f"{name}: rel_l2 {r:.3e} cos {c:.7f}"


def test_dequant_mxfp4_bit_exact(dev):
    from int4_quantized_moe_amd import _lib

    _say("dequant: every byte at in-domain scales 2^-13 .. 2^13 and zero")
    n, k = 27, 256
    packed = np.tile(np.arange(256, dtype=np.uint8).reshape(2, 128), (n // 2 + 1, 1))[:n].copy()
    exps = np.arange(114, 141)  # 2^-13 .. 2^13, one per row
    scales = W.ue8m0_to_bf16_bits(np.repeat(exps[:, None], k // 32, axis=1))
    scales[3, 2] = 0  # UE8M0 0 bit-casts to +0
    out = torch.empty((n, k), dtype=torch.float32, device="cuda")
    _lib.kt_rawint4_dequant_mxfp4(torch.from_numpy(packed).cuda(), dev.bf16_tensor(scales, "cuda"), n, k, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = O.dequant(packed, scales, "mxfp4")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _run(dev, cfg, weights, batch, grad_scale=1.0):
    dl = dev.DeviceLayer(cfg, weights)
    db = dev.DeviceBatch(batch)
    ws = dl.workspace(db.qlen)
    out = dl.forward(db.inputs, db.expert_ids, db.route_weights, ws)
    pre_g, pre_u = dl.saved_preactivations(db.qlen, ws)
    grads = dl.grad_buffers(fill=7.0)
    droute = torch.empty(batch.expert_ids.shape, dtype=torch.float32, device="cuda")
    dx, _ = dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, grads, accumulate=False,
                        grad_scale=grad_scale, grad_route=droute)
    torch.cuda.synchronize()
    bad_ids, bad_scales = __import__("int4_quantized_moe_amd")._lib.kt_rawint4_moe_diagnostics(ws)
    assert bad_ids == 0 and bad_scales == 0
    return dl, {"out": out.float().cpu().numpy(), "dx": dx.float().cpu().numpy(), "droute": droute.cpu().numpy(),
                "grads": {n: g.cpu().numpy() for n, g in grads.items()},
                "sides": (pre_g.cpu().numpy(), pre_u.cpu().numpy())}


def _check(tag, cfg, weights, batch, gpu, grad_scale=1.0):
    ref = reference(cfg, weights, batch.inputs, batch.expert_ids, batch.route_weights, batch.grad_output,
                    gpu["sides"], _say)
    checks = [("forward", gpu["out"], ref["out"], REL_L2, COSINE), ("dX", gpu["dx"], ref["dx"], REL_L2, COSINE),
              ("dRoute", gpu["droute"], ref["droute"], DROUTE_REL_L2, 0.995)]
    checks += [(n, gpu["grads"][n], grad_scale * ref["grads"][n], REL_L2, COSINE) for n in O.LORA_NAMES]
    failures = []
    for name, a, e, rel, cos in checks:
        try:
            _close(f"{tag}.{name}", a, e, rel, cos)
        except AssertionError as err:
            failures.append(str(err))
    assert not failures, "; ".join(failures)
    active = set(batch.expert_ids.ravel().tolist())
    for n in O.LORA_NAMES:
        for e in range(gpu["grads"][n].shape[0]):
            if e not in active:
                assert np.count_nonzero(gpu["grads"][n][e]) == 0, f"{tag}.{n}: stale rows for expert {e}"


@pytest.mark.parametrize("index", [0, 1])
def test_mxfp4_layer_small_configs(dev, index):
    cfg = _mx(W.CONFIGS[index])
    _say("layer", cfg.name)
    weights = W.make_weights(cfg, W.config_seed(index))
    batch = W.make_batch(cfg, W.config_seed(index))
    before = O.base_storage_hash(weights)
    _, gpu = _run(dev, cfg, weights, batch, grad_scale=0.5)
    _check(cfg.name, cfg, weights, batch, gpu, grad_scale=0.5)
    assert O.base_storage_hash(weights) == before


def _heights_case(rank):
    if rank == 6:
        cfg = W.LayerConfig("heights_mxfp4", 5, 2, 160, 224, 6, 12.0, 180, 2.5, x_std=2.0, weight_format="mxfp4")
        weights, batch = W.make_weights(cfg, 91), W.make_batch(cfg, 91)
        batch.expert_ids[:150, 0] = 1
        batch.expert_ids[:150, 1] = np.where(batch.expert_ids[:150, 1] == 1, 3, batch.expert_ids[:150, 1])
    else:
        cfg = W.LayerConfig("heights64_mxfp4", 4, 2, 256, 192, 64, 128.0, 264, 3.0, x_std=2.0, weight_format="mxfp4")
        weights, batch = W.make_weights(cfg, 93), W.make_batch(cfg, 93)
        ids = batch.expert_ids
        ids[:, 1] = np.where(ids[:, 1] == 1, ids[:, 0], ids[:, 1])
        ids[:, 0] = 1
        ids[:, 1] = np.where(ids[:, 1] == 1, 3, ids[:, 1])
    return cfg, weights, batch


@pytest.mark.parametrize("rank", [6, 64])
@pytest.mark.parametrize("rows", [16, 32, 64, 96, 128, 0])
def test_mxfp4_every_tile_height(dev, rank, rows, monkeypatch):
    cfg, weights, batch = _heights_case(rank)
    _say("tile height", rows or "mixed", "rank", rank)
    if rows:
        monkeypatch.setenv("KT_RAWINT4_GEMM_ROWS", str(rows))
    else:
        monkeypatch.delenv("KT_RAWINT4_GEMM_ROWS", raising=False)
    _, gpu = _run(dev, cfg, weights, batch)
    _check(f"r{rank}rows{rows or 'mixed'}", cfg, weights, batch, gpu)


def test_mxfp4_inference_base_only(dev):
    cfg = _mx(W.CONFIGS[1])
    _say("inference, base alone", cfg.name)
    weights = W.make_weights(cfg, 21)
    batch = W.make_batch(cfg, 21)
    dl = dev.DeviceLayer(cfg, weights, base_only=True)
    db = dev.DeviceBatch(batch)
    out = dl.infer(db.inputs, db.expert_ids, db.route_weights, dl.infer_workspace(db.qlen))
    torch.cuda.synchronize()
    zero = {n: np.zeros(s) for n, s in cfg.lora_shapes().items()}
    ref = O.moe(cfg, weights, batch.inputs, batch.expert_ids, batch.route_weights, lora=zero)
    _close(f"{cfg.name}.base", out.float().cpu().numpy(), ref["out"])


def test_mxfp4_scales_outside_the_domain_are_counted(dev):
    cfg = _mx(W.CONFIGS[0])
    _say("scale domain", cfg.name)
    weights = W.make_weights(cfg, 5)
    batch = W.make_batch(cfg, 5)
    used = int(batch.expert_ids[0, 0])
    weights.gate_scale[used, 0, 0] = W.f32_to_bf16_bits(np.array([0.75], dtype=np.float32))[0]  # not a power of two
    weights.down_scale[used, 1, 0] = W.ue8m0_to_bf16_bits(np.array([122]))[0] | 0x8000  # -2^-5: has a sign
    weights.up_scale[used, 2, 1] = W.ue8m0_to_bf16_bits(np.array([113]))[0]  # 2^-14: shifted into the domain
    dl = dev.DeviceLayer(cfg, weights)
    db = dev.DeviceBatch(batch)
    ws = dl.workspace(db.qlen)
    dl.forward(db.inputs, db.expert_ids, db.route_weights, ws)
    torch.cuda.synchronize()
    _, bad_scales = __import__("int4_quantized_moe_amd")._lib.kt_rawint4_moe_diagnostics(ws)
    assert bad_scales == 2  # the scale that is not a power of two and the signed one


def test_mxfp4_full_size_sampled(dev):
    # sampled tokens and experts of the long-sequence workload with an MXFP4 base
    # (tests/fullsize.py: the heaviest, the lightest and one expert of every
    # last-tile height class)
    base = W.CONFIGS[4]
    cfg = _mx(base)
    seed = W.config_seed(4)
    _say(f"{cfg.name}: generating")
    weights = W.make_weights(cfg, seed)
    batch = W.make_batch(cfg, seed)
    _say(f"{cfg.name}: forward + backward on the GPU")
    dl = dev.DeviceLayer(cfg, weights)
    db = dev.DeviceBatch(batch)
    ws = dl.workspace(db.qlen)
    out = dl.forward(db.inputs, db.expert_ids, db.route_weights, ws)
    pre_g, pre_u = dl.saved_preactivations(db.qlen, ws)
    grads = dl.grad_buffers(fill=7.0)
    droute = torch.empty(batch.expert_ids.shape, dtype=torch.float32, device="cuda")
    dx, _ = dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, grads, accumulate=False,
                        grad_scale=1.0, grad_route=droute)
    torch.cuda.synchronize()
    bad_ids, bad_scales = __import__("int4_quantized_moe_amd")._lib.kt_rawint4_moe_diagnostics(ws)
    assert bad_ids == 0 and bad_scales == 0

    def sides(rows):
        index = torch.from_numpy(rows).cuda()
        return pre_g[index].cpu().numpy(), pre_u[index].cpu().numpy()

    rng = np.random.default_rng(6262)
    toks = np.unique(np.concatenate([[0, cfg.qlen - 1], rng.choice(cfg.qlen, 6, replace=False)]))
    failures = F.check_tokens(cfg, weights, batch, out.float().cpu().numpy(), dx.float().cpu().numpy(),
                              droute.cpu().numpy(), sides, toks, _say)
    g = {n: t.cpu().numpy() for n, t in grads.items()}
    counts = np.bincount(batch.expert_ids.ravel(), minlength=cfg.num_experts)
    experts = F.choose_experts(counts, rng, n=4)
    failures += F.check_experts(cfg, weights, batch, g, sides, experts, _say)
    assert not failures, "; ".join(failures)


def test_mxfp4_zipf_full_size_recompute_and_inference(dev):
    # the Zipf-routed workload (one expert with ~3500 rows) with an MXFP4 base:
    # inference + recompute backward equal forward + backward bit for bit, and
    # sampled tokens of the forward match the oracle
    cfg = _mx(W.CONFIGS[3])
    seed = W.config_seed(3)
    _say(f"{cfg.name}: generating")
    weights = W.make_weights(cfg, seed)
    batch = W.make_batch(cfg, seed)
    dl = dev.DeviceLayer(cfg, weights)
    db = dev.DeviceBatch(batch)

    def bits(t):
        return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()

    _say(f"{cfg.name}: forward + backward")
    ws = dl.workspace(db.qlen)
    out = dl.forward(db.inputs, db.expert_ids, db.route_weights, ws)
    g_ref = dl.grad_buffers(fill=0.0)
    dx_ref, _ = dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, g_ref)
    _say(f"{cfg.name}: inference + recompute backward")
    out_inf = dl.infer(db.inputs, db.expert_ids, db.route_weights, dl.infer_workspace(db.qlen))
    ws.fill_(0xFF)
    g = dl.grad_buffers(fill=0.0)
    dx, _ = dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, g, recompute=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out_inf), bits(out))
    assert np.array_equal(bits(dx), bits(dx_ref))
    for n in O.LORA_NAMES:
        assert np.array_equal(bits(g[n]), bits(g_ref[n])), n
    rng = np.random.default_rng(7373)
    toks = np.unique(np.concatenate([[0, cfg.qlen - 1], rng.choice(cfg.qlen, 6, replace=False)]))
    _say(f"{cfg.name}: oracle forward on tokens {toks.tolist()}")
    ref = O.moe(cfg, weights, batch.inputs[toks], batch.expert_ids[toks], batch.route_weights[toks])
    _close(f"{cfg.name}.forward", out.float().cpu().numpy()[toks], ref["out"])
