"""GPU: no kernel writes outside its outputs.

Every buffer the library writes (output, grad_input, grad_route, the six
gradient buffers, the workspace) is carved out of a larger allocation whose
guard regions before and after hold a fixed byte pattern; after training
forward + backward, the inference forward and the recompute backward (RAWINT4
and MXFP4, several tile heights at once) every guard byte must be unchanged.
Each case prints its name first.
"""


import numpy as np
import pytest

from int4_quantized_moe_amd import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side
PATTERN = 0xA5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int4_quantized_moe_amd import device

    return device


def _say(*a):
    print("[canary]", *a, flush=True)


class Guarded:
    """A byte buffer with guard regions; .view(dtype, shape) is the usable middle."""

    def __init__(self, nbytes):
        self.nbytes = nbytes
        self.raw = torch.full((GUARD + nbytes + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")

    def view(self, dtype, shape):
        return self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(shape)

    def intact(self):
        head = self.raw[:GUARD].cpu().numpy()
        tail = self.raw[GUARD + self.nbytes:].cpu().numpy()
        return bool((head == PATTERN).all() and (tail == PATTERN).all())


def _case(fmt):
    cfg = W.LayerConfig(f"canary_{fmt}", 5, 2, 160, 224, 8, 12.0, 180, 2.5, x_std=2.0, weight_format=fmt)
    weights = W.make_weights(cfg, 95)
    batch = W.make_batch(cfg, 95)
    batch.expert_ids[:150, 0] = 1  # one expert over several tile heights
    batch.expert_ids[:150, 1] = np.where(batch.expert_ids[:150, 1] == 1, 3, batch.expert_ids[:150, 1])
    return cfg, weights, batch


@pytest.mark.parametrize("fmt", ["rawint4", "mxfp4"])
def test_guards_stay_intact(dev, fmt):
    cfg, weights, batch = _case(fmt)
    _say(cfg.name)
    dl = dev.DeviceLayer(cfg, weights)
    db = dev.DeviceBatch(batch)
    q, h, k = db.qlen, cfg.hidden, cfg.top_k
    bufs = {"out": Guarded(q * h * 2), "dx": Guarded(q * h * 2), "droute": Guarded(q * k * 4),
            "ws": Guarded(dl.workspace(q).numel()), "wsi": Guarded(dl.infer_workspace(q).numel()),
            "outi": Guarded(q * h * 2)}
    shapes = cfg.lora_shapes()
    for n, s in shapes.items():
        bufs[n] = Guarded(int(np.prod(s)) * 4)
    out = bufs["out"].view(torch.bfloat16, (q, h))
    dx = bufs["dx"].view(torch.bfloat16, (q, h))
    dr = bufs["droute"].view(torch.float32, (q, k))
    ws = bufs["ws"].view(torch.uint8, (-1,))
    grads = {n: bufs[n].view(torch.float32, shapes[n]) for n in shapes}
    for g in grads.values():
        g.zero_()
    dl.forward(db.inputs, db.expert_ids, db.route_weights, ws, output=out)
    dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, grads, accumulate=True,
                grad_scale=0.5, grad_input=dx, grad_route=dr)
    dl.infer(db.inputs, db.expert_ids, db.route_weights, bufs["wsi"].view(torch.uint8, (-1,)),
             output=bufs["outi"].view(torch.bfloat16, (q, h)))
    dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, grads, accumulate=False,
                grad_scale=1.0, grad_input=dx, grad_route=dr, recompute=True)
    torch.cuda.synchronize()
    broken = [n for n, b in bufs.items() if not b.intact()]
    assert not broken, f"guard bytes changed around {broken}"
    assert torch.isfinite(out.float()).all() and torch.isfinite(dx.float()).all()
