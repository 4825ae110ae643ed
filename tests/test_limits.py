"""GPU parity at the ABI's limits: the largest rank (128, both LoRA halves of
gate/up 128 wide), the largest expert count (8192, most experts empty, a few
ids at the top of the range), and top_k = num_experts.  Oracle and bars as in
test_parity.  Each case prints its name first.  Also more than eight slots
per token, which the output and dx combine read in rounds of eight."""

import numpy as np
import pytest

import oracle as O
from int4_quantized_moe_amd import workloads as W
from tests.clamp_sides import reference

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_quantized_moe_amd import device

    return device


def _say(*a):
    print("[limits]", *a, flush=True)


def _run_and_check(dev, cfg, weights, batch):
    dl = dev.DeviceLayer(cfg, weights)
    db = dev.DeviceBatch(batch)
    ws = dl.workspace(db.qlen)
    out = dl.forward(db.inputs, db.expert_ids, db.route_weights, ws)
    pre = dl.saved_preactivations(db.qlen, ws)
    grads = dl.grad_buffers(fill=7.0)
    dr = torch.empty(batch.expert_ids.shape, dtype=torch.float32, device="cuda")
    dx, _ = dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, grads, grad_route=dr)
    torch.cuda.synchronize()
    ref = reference(cfg, weights, batch.inputs, batch.expert_ids, batch.route_weights, batch.grad_output,
                    tuple(t.cpu().numpy() for t in pre), _say)
    checks = [("forward", out.float().cpu().numpy(), ref["out"], 5e-3, 0.9999),
              ("dX", dx.float().cpu().numpy(), ref["dx"], 5e-3, 0.9999),
              ("dRoute", dr.cpu().numpy(), ref["droute"], 3e-2, 0.995)]
    g = {n: t.cpu().numpy() for n, t in grads.items()}
    ids = batch.expert_ids
    active = np.unique(ids[(ids >= 0) & (ids < cfg.num_experts)])
    checks += [(n, g[n][active], ref["grads"][n][active], 5e-3, 0.9999) for n in O.LORA_NAMES]
    failures = []
    for name, a, e, rel, cos in checks:
        r, c = O.relative_l2_and_cosine(np.asarray(a, np.float64), e)
        _say(f"{cfg.name}.{name}: rel_l2={r:.3e} cos={c:.7f}")
        if not (np.isfinite(a).all() and r <= rel and c >= cos):
            failures.append(f"{name}: rel_l2 {r:.3e} cos {c:.7f}")
    assert not failures, "; ".join(failures)
    idle = np.setdiff1d(np.arange(cfg.num_experts), active)
    for n in O.LORA_NAMES:
        assert np.count_nonzero(g[n][idle]) == 0, f"{cfg.name}.{n}: idle experts have gradients"


@pytest.mark.parametrize("rows", [0, 16])
def test_rank_128(dev, rows, monkeypatch):
    cfg = W.LayerConfig("rank128", 4, 2, 256, 192, 128, 64.0, 150, 2.0, x_std=2.0)
    _say("rank 128, tile rows", rows or "default")
    if rows:
        monkeypatch.setenv("KT_RAWINT4_GEMM_ROWS", str(rows))
    else:
        monkeypatch.delenv("KT_RAWINT4_GEMM_ROWS", raising=False)
    _run_and_check(dev, cfg, W.make_weights(cfg, 131), W.make_batch(cfg, 131))


def test_max_experts(dev):
    cfg = W.LayerConfig("experts8192", 8192, 4, 64, 64, 4, 8.0, 40, 1.0, x_std=2.0)
    _say("8192 experts")
    weights = W.make_weights(cfg, 133)
    batch = W.make_batch(cfg, 133)
    batch.expert_ids[0] = [8191, 8190, 0, 4096]  # the top of the range and the bottom
    batch.expert_ids[1] = [8191, 1, 2, 3]
    assert all(len(set(r)) == 4 for r in batch.expert_ids.tolist())
    _run_and_check(dev, cfg, weights, batch)


def test_top_k_equals_experts(dev):
    cfg = W.LayerConfig("topk_all", 6, 6, 96, 128, 8, 16.0, 20, 0.0)
    _say("top_k = num_experts")
    _run_and_check(dev, cfg, W.make_weights(cfg, 137), W.make_batch(cfg, 137))


def test_top_k_above_eight_with_dropped_slots(dev):
    # 12 slots per token: the combine sums them in two rounds (8 + 4); some slots
    # of both rounds carry dropped ids (-1, or past the last expert), which add nothing
    cfg = W.LayerConfig("topk12", 20, 12, 96, 128, 8, 16.0, 24, 1.5, x_std=2.0)
    _say("top_k = 12 with dropped slots")
    weights = W.make_weights(cfg, 139)
    batch = W.make_batch(cfg, 139)
    batch.expert_ids[0, 9] = -1
    batch.expert_ids[1, 3] = cfg.num_experts
    batch.expert_ids[2, 11] = -1
    batch.expert_ids[2, 10] = cfg.num_experts + 5
    batch.expert_ids[5, 8:] = -1
    _run_and_check(dev, cfg, weights, batch)
