"""GPU parity at the full benchmark sizes, in the launch configuration bench.py times.

The two large workloads (384 experts, top-8, hidden 7168, intermediate 2048;
4096 Zipf-routed tokens at rank 16 and 16384 uniformly routed tokens at rank
64 with the clamp at 7) run once each through the C ABI with the default tile
choice; the oracle then checks what it can compute piece by piece
(tests/fullsize.py): sampled tokens with the oracle's own clamp masks, and the
six LoRA gradients of at least eight sampled experts -- the heaviest, the
lightest, one of every height class of the last row tile -- each with the GPU's
clamp side taken only within the a priori error bound of a bound, all of them
together with the oracle's own masks.  Experts no slot reaches must have
exactly zero gradients.

Bars as in test_parity: relative L2 <= 5e-3 and cosine >= 0.9999 (dRoute
3e-2).  Each step prints what it does first.
"""

import numpy as np
import pytest

import oracle as O
from int4_quantized_moe_amd import workloads as W
from tests import fullsize as F

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

N_TOKENS = 8


def _say(*a):
    print("[parity-full]", *a, flush=True)


@pytest.fixture(scope="module", params=[3, 4], ids=["k2_qlen4096_zipf", "k2_qlen16384_r64"])
def full(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_quantized_moe_amd import _lib, device

    index = request.param
    _say(f"{W.CONFIGS[index].name}: generating")
    cfg, weights, batch = W.make_workload(index)
    _say(f"{cfg.name}: forward + backward on the GPU")
    dl = device.DeviceLayer(cfg, weights)
    db = device.DeviceBatch(batch)
    ws = dl.workspace(db.qlen)
    out = dl.forward(db.inputs, db.expert_ids, db.route_weights, ws)
    pre_g, pre_u = dl.saved_preactivations(db.qlen, ws)
    grads = dl.grad_buffers(fill=7.0)
    droute = torch.empty(batch.expert_ids.shape, dtype=torch.float32, device="cuda")
    dx, _ = dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, grads, accumulate=False,
                        grad_scale=1.0, grad_route=droute)
    torch.cuda.synchronize()
    bad_ids, bad_scales = _lib.kt_rawint4_moe_diagnostics(ws)
    assert bad_ids == 0 and bad_scales == 0
    del ws

    def sides(rows):
        index = torch.from_numpy(rows).cuda()
        return pre_g[index].cpu().numpy(), pre_u[index].cpu().numpy()

    res = {"index": index, "cfg": cfg, "weights": weights, "batch": batch, "sides": sides,
           "out": out.float().cpu().numpy(), "dx": dx.float().cpu().numpy(), "droute": droute.cpu().numpy(),
           "grads": {n: t.cpu().numpy() for n, t in grads.items()}}
    yield res
    del pre_g, pre_u


def test_full_size_sampled_tokens(full):
    cfg, batch = full["cfg"], full["batch"]
    rng = np.random.default_rng(4242 + full["index"])
    toks = np.unique(np.concatenate([[0, cfg.qlen - 1], rng.choice(cfg.qlen, N_TOKENS, replace=False)]))
    failures = F.check_tokens(cfg, full["weights"], batch, full["out"], full["dx"], full["droute"], full["sides"],
                              toks, _say)
    assert not failures, "; ".join(failures)


def test_full_size_sampled_experts(full):
    cfg, batch = full["cfg"], full["batch"]
    counts = np.bincount(batch.expert_ids.ravel(), minlength=cfg.num_experts)
    experts = F.choose_experts(counts, np.random.default_rng(5151 + full["index"]))
    _say(f"{cfg.name}: experts {experts} (slots {counts[experts].tolist()})")
    assert len(experts) >= 8
    failures = F.check_experts(cfg, full["weights"], batch, full["grads"], full["sides"], experts, _say)
    assert not failures, "; ".join(failures)


def test_full_size_inactive_experts_zero(full):
    cfg, batch, g = full["cfg"], full["batch"], full["grads"]
    counts = np.bincount(batch.expert_ids.ravel(), minlength=cfg.num_experts)
    _say(f"{cfg.name}: {int(np.count_nonzero(counts == 0))} experts without a slot")
    for e in np.flatnonzero(counts == 0):
        for n in O.LORA_NAMES:
            assert np.count_nonzero(g[n][e]) == 0, f"{cfg.name}.{n}: expert {e} has no slot but a gradient"
    # every expert with slots has its gradients written (none left whole at the 7.0 fill)
    for e in np.flatnonzero(counts):
        for n in O.LORA_NAMES:
            assert not np.all(g[n][e] == 7.0), f"{cfg.name}.{n}: expert {e} kept the fill value"
