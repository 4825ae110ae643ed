"""The oracle as the parity reference of a GPU run, and clamp masks at their bounds.

The SwiGLU clamp's masks are discontinuous at g = L and u = -L, L.  The GPU sums a
pre-activation in fp32 in its own order, the oracle in double (rounded to fp32
once), so a value on a bound to within that rounding can fall on either side, and
either mask is then a correct result.

``reference`` is the plain check: the oracle decides every mask on its own
values.  When the GPU's saved pre-activations (the values its masks were decided
on) are given, each must lie within the oracle's a priori bound on the error of
an fp32 computation of it (the oracle's ``preact_bound``: exact base products,
LoRA factors to 2^-13, fp32 sums by the probabilistic bound of Higham and Mary);
that is checked element by element and is all the GPU values are used for.

``reference_decided`` is for the full-size sampled checks only, where a single
element within rounding of a bound moves its expert's gate/up LoRA gradients by a
few 1e-3: within each element's a priori bound of a bound the oracle takes the
GPU's side (the oracle's decided mode), everywhere else its own.  It reports how
many elements are that close and how many of them end with a decision other than
the oracle's own, and caps the latter.
"""

import numpy as np

import oracle as O


def _valid(cfg, ids):
    return (ids >= 0) & (ids < cfg.num_experts)


def _check_sides(cfg, ref, sides, valid, say, tag):
    g, u = (np.asarray(a, dtype=np.float64).reshape(ref["pre_g"].shape) for a in sides)
    dg = np.abs(g - ref["pre_g"])[valid]
    du = np.abs(u - ref["pre_u"])[valid]
    bg, bu = ref["bound_g"][valid], ref["bound_u"][valid]
    worst = max(float((dg / bg).max(initial=0.0)), float((du / bu).max(initial=0.0)))
    say(f"{tag}pre-activations: max |gpu - oracle| g {dg.max(initial=0.0):.2e} u {du.max(initial=0.0):.2e}; "
        f"largest share of the a priori bound {worst:.3f}")
    assert np.all(dg <= bg) and np.all(du <= bu), f"saved pre-activations beyond the a priori bound ({worst:.3f}x)"
    return g, u


def reference(cfg, weights, inputs, ids, rw, dy, sides, say, tag=""):
    """The oracle with its own masks; the GPU's pre-activations (if given) checked against it."""
    ref = O.moe(cfg, weights, inputs, ids, rw, dy, preactivations=True)
    if sides is not None:
        _check_sides(cfg, ref, sides, _valid(cfg, ids), say, tag)
    return ref


def _masks(limit, g, u):
    return g <= limit, (u >= -limit) & (u <= limit)


def reference_decided(cfg, weights, inputs, ids, rw, dy, sides, say, tag="", cap=None):
    """The oracle taking the GPU's side within each element's a priori bound of a clamp
    bound; returns it and the number of masks that ended on a side other than the
    oracle's own (zero: the result equals the plain ``reference``)."""
    ref = O.moe(cfg, weights, inputs, ids, rw, dy, sides=sides, band=O.APRIORI, preactivations=True)
    valid = _valid(cfg, ids)
    g, u = _check_sides(cfg, ref, sides, valid, say, tag)
    lim = cfg.swiglu_limit
    flipped = 0
    if lim > 0:
        pg, pu, bg, bu = (ref[k][valid] for k in ("pre_g", "pre_u", "bound_g", "bound_u"))
        near_g = np.abs(pg - lim) <= bg
        near_u = (np.abs(pu - lim) <= bu) | (np.abs(pu + lim) <= bu)
        own_g, own_u = _masks(lim, pg, pu)
        gpu_g, gpu_u = _masks(lim, g[valid], u[valid])
        flipped = int(np.count_nonzero(near_g & (own_g != gpu_g)) + np.count_nonzero(near_u & (own_u != gpu_u)))
        n = 2 * pg.size
        limit = cap if cap is not None else max(8, int(1e-5 * n))
        say(f"{tag}clamp sides: {int(near_g.sum() + near_u.sum())} of {n} masks within the a priori bound of a "
            f"bound; {flipped} take the GPU's other side (at most {limit})")
        assert flipped <= limit, f"{flipped} masks decided on the GPU's side (cap {limit})"
    return ref, flipped
