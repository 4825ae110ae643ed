"""Clamp masks at their bounds: the side the GPU took, checked, handed to the oracle.

The SwiGLU clamp's masks are discontinuous at g = L and u = -L, L.  The GPU sums
the pre-activations in fp32 in its own order, the oracle in double; a value on a
bound to within that rounding can fall on either side, and either mask is then a
correct result -- but one flipped element moves a token's grad_input by about
1/sqrt(unmasked elements) and its expert's gate/up LoRA gradients by a few
1e-3, which the parity bars would count as an error.  So:

* the GPU's saved pre-activations (what its masks were decided on) must agree
  with the oracle's to within a band of 2^-16 times their largest magnitude,
  element by element, on every valid slot;
* inside that band of a bound the oracle takes the GPU's side (the oracle's
  documented decided mode); everywhere else it decides on its own value.
"""

import numpy as np

import oracle as O

BAND = 2.0 ** -16  # relative to the largest pre-activation magnitude


def reference(cfg, weights, inputs, ids, rw, dy, sides, say):
    g, u = (np.asarray(a, dtype=np.float64) for a in sides)
    valid = (ids >= 0) & (ids < cfg.num_experts)
    scale = max(float(np.abs(g[valid]).max(initial=0.0)), float(np.abs(u[valid]).max(initial=0.0)), 1.0)
    band = BAND * scale
    ref = O.moe(cfg, weights, inputs, ids, rw, dy, sides=(g, u), band=band, preactivations=True)
    dg = float(np.abs(g[valid] - ref["pre_g"][valid]).max(initial=0.0))
    du = float(np.abs(u[valid] - ref["pre_u"][valid]).max(initial=0.0))
    near = 0
    if cfg.swiglu_limit > 0:
        lim = cfg.swiglu_limit
        near = int(np.count_nonzero(np.abs(ref["pre_g"][valid] - lim) <= band)
                   + np.count_nonzero(np.minimum(np.abs(ref["pre_u"][valid] - lim),
                                                 np.abs(ref["pre_u"][valid] + lim)) <= band))
    say(f"pre-activations: max |gpu - oracle| g {dg:.2e} u {du:.2e}, band {band:.2e}, {near} within it of a bound")
    assert dg <= band and du <= band, f"saved pre-activations off by {max(dg, du):.3e} (band {band:.3e})"
    return ref
