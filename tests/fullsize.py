"""Parity at the full benchmark sizes on samples the oracle can compute piece by piece.

* Sampled tokens: a token's output, grad_input and grad_route depend only on its
  own input, routing and output gradient, so the oracle runs on those tokens
  alone, deciding every clamp mask on its own values.
* Sampled experts: an expert's six LoRA gradients sum over exactly the slots
  routed to it, so the oracle runs on the tokens that reach it with every other
  slot dropped (id -1).  The sample holds the heaviest and the lightest expert,
  one expert of every height class of the GEMMs' last row tile (16, 32, 64, 96
  or 128 rows, where present) and random others, at least ``n`` in all.  Each
  expert is held to the bar with the oracle taking the GPU's clamp side within
  the a priori bound of a bound (tests/clamp_sides.py); all sampled experts
  together are held to it with the oracle's own masks.
"""

import numpy as np

import oracle as O

from tests.clamp_sides import reference, reference_decided

REL_L2 = 5e-3
COSINE = 0.9999
DROUTE_REL_L2 = 3e-2
BULK = 128  # full GEMM row tile
CLASSES = (16, 32, 64, 96, 128)


def last_tile_height(count):
    """Height of the tile that holds an expert's last rows: full 128-row tiles first,
    then the smallest class that holds the rest."""
    rest = count - BULK * ((count - 1) // BULK)
    return next(h for h in CLASSES if rest <= h)


def choose_experts(counts, rng, n=8):
    used = np.flatnonzero(counts)
    picks = [int(used[np.argmax(counts[used])]), int(used[np.argmin(counts[used])])]
    for h in CLASSES:
        cls = [int(e) for e in used if last_tile_height(int(counts[e])) == h and int(e) not in picks]
        if cls:
            picks.append(int(rng.choice(cls)))
    rest = [int(e) for e in used if int(e) not in picks]
    while len(picks) < n and rest:
        picks.append(rest.pop(int(rng.integers(len(rest)))))
    return picks


def close(say, name, actual, expected, rel=REL_L2, cos=COSINE):
    a = np.asarray(actual, dtype=np.float64)
    e = np.asarray(expected, dtype=np.float64)
    assert np.isfinite(a).all(), f"{name}: non-finite values"
    assert np.count_nonzero(e), f"{name}: reference has no signal"
    r, c = O.relative_l2_and_cosine(a, e)
    say(f"{name}: rel_l2={r:.3e} cos={c:.7f}")
    assert r <= rel and c >= cos, f"{name}: rel_l2 {r:.3e} cos {c:.7f}"


def _collect(failures, fn, *args, **kw):
    try:
        fn(*args, **kw)
    except AssertionError as err:
        failures.append(str(err))


def check_tokens(cfg, weights, batch, out, dx, droute, sides, toks, say):
    """Failures of the sampled tokens (out, dx, droute: the GPU's whole arrays; sides(rows))."""
    say(f"{cfg.name}: oracle on tokens {toks.tolist()}")
    ref = reference(cfg, weights, batch.inputs[toks], batch.expert_ids[toks], batch.route_weights[toks],
                    batch.grad_output[toks], sides(toks), say, tag=f"{cfg.name}.tokens ")
    failures = []
    _collect(failures, close, say, f"{cfg.name}.forward", out[toks], ref["out"])
    if dx is not None:
        _collect(failures, close, say, f"{cfg.name}.dX", dx[toks], ref["dx"])
        _collect(failures, close, say, f"{cfg.name}.dRoute", droute[toks], ref["droute"], DROUTE_REL_L2, 0.995)
    return failures


def check_experts(cfg, weights, batch, grads, sides, experts, say):
    """Failures of the sampled experts' LoRA gradients (grads: the GPU's, numpy, by name)."""
    failures = []
    mine = {n: [] for n in O.LORA_NAMES}
    want = {n: [] for n in O.LORA_NAMES}
    counts = np.bincount(batch.expert_ids[(batch.expert_ids >= 0) & (batch.expert_ids < cfg.num_experts)],
                         minlength=cfg.num_experts)
    for e in experts:
        rows = np.flatnonzero((batch.expert_ids == e).any(axis=1))
        ids = np.where(batch.expert_ids[rows] == e, e, -1).astype(np.int64)
        say(f"{cfg.name}: oracle LoRA gradients of expert {e} ({counts[e]} slots, last tile "
            f"{last_tile_height(int(counts[e]))} rows)")
        args = (cfg, weights, batch.inputs[rows], ids, batch.route_weights[rows], batch.grad_output[rows])
        ref, flipped = reference_decided(*args, sides(rows), say, tag=f"{cfg.name}.expert{e} ")
        for n in O.LORA_NAMES:
            _collect(failures, close, say, f"{cfg.name}.expert{e}.{n}", grads[n][e], ref["grads"][n][e])
        own = ref if flipped == 0 else reference(*args, None, say)
        for n in O.LORA_NAMES:
            mine[n].append(grads[n][e].ravel())
            want[n].append(own["grads"][n][e].ravel())
    for n in O.LORA_NAMES:
        _collect(failures, close, say, f"{cfg.name}.experts{len(experts)}.{n} (own masks)",
                 np.concatenate(mine[n]), np.concatenate(want[n]))
    return failures
