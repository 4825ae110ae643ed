"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each check ties the oracle to something other than itself: values printed on the
pages (fixtures under tests/golden/), closed forms of hand-built cases, a
textbook special case computed by torch, autograd of the same equation,
finite differences, matrix identities and invariants.  Runs on the CPU only.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from int4_quantized_moe_amd import workloads as W

BF16_HALF = 0x3F00  # 0.5
BF16_ONE = 0x3F80  # 1.0
BF16_SIXTEENTH = 0x3D80  # 0.0625


def _cfg(e, k, h, i, r, alpha, qlen, limit, name="t"):
    return W.LayerConfig(name, e, k, h, i, r, float(alpha), qlen, float(limit))


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _silu(z):
    return z * _sig(z)


def _dsilu(z):
    s = _sig(z)
    return s * (1.0 + z * (1.0 - s))


# ------------------------------------------------------------------ codec


def test_unpack_matches_page_fixtures(golden):
    for byte, v0, v1 in golden("codec_extremes.txt"):
        assert O.unpack(np.array([int(byte, 16)], dtype=np.uint8)).tolist() == [int(v0), int(v1)]


def test_pack_unpack_round_trip_all_bytes():
    every = np.arange(256, dtype=np.uint8).reshape(16, 16)
    codes = O.unpack(every).astype(np.int32) + 8
    assert codes.min() == 0 and codes.max() == 15
    assert np.array_equal(O.pack(codes), every)


def test_pack_rejects_bad_codes():
    with pytest.raises(ValueError, match="even"):
        O.pack(np.zeros(3, dtype=np.int32))
    with pytest.raises(ValueError, match=r"\[0, 15\]"):
        O.pack(np.array([0, 16], dtype=np.int32))
    with pytest.raises(ValueError, match=r"\[0, 15\]"):
        O.pack(np.array([-1, 3], dtype=np.int32))


def test_layout_validation(golden):
    rows = dict((r[0], r[1]) for r in golden("layout.txt"))
    assert int(rows["group_size"]) == 32
    packed = np.zeros((4, 16), dtype=np.uint8)
    scales = np.zeros((4, 1), dtype=np.uint16)
    assert O.validate_layout(packed, scales) == (4, 32)
    with pytest.raises(ValueError, match="group_size"):
        O.validate_layout(packed, scales, group_size=16)
    with pytest.raises(ValueError, match="divisible"):
        O.validate_layout(np.zeros((4, 17), dtype=np.uint8), np.zeros((4, 1), dtype=np.uint16))
    with pytest.raises(ValueError, match="shape"):
        O.validate_layout(packed, np.zeros((4, 2), dtype=np.uint16))
    with pytest.raises(ValueError, match="uint8"):
        O.validate_layout(packed.astype(np.int16), scales)
    with pytest.raises(ValueError, match="bf16"):
        O.validate_layout(packed, scales.astype(np.float32))


def test_dequant_fixture_values_and_zero_scale():
    # one row of two groups: group 0 bytes 0x00 (-8,-8) and 0xFF (+7,+7) at scale
    # 0.0625; group 1 random codes with a zero scale, which the format allows
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x00
    packed[0, 1] = 0xFF
    packed[0, 2] = 0x21
    packed[0, 16:] = np.arange(16, dtype=np.uint8) * 17 + 3
    scales = np.array([[BF16_SIXTEENTH, 0x0000]], dtype=np.uint16)
    w = O.dequant(packed, scales)
    assert w[0, :6].tolist() == [-0.5, -0.5, 0.4375, 0.4375, -0.4375, -0.375]
    assert np.all(w[0, 6:32] == -0.5)  # bytes 0 decode to -8 each
    assert np.all(w[0, 32:] == 0.0)


def test_dequant_group_indexing():
    rng = np.random.default_rng(5)
    packed = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    ones = np.full((3, 4), BF16_ONE, dtype=np.uint16)
    base = O.dequant(packed, ones)
    # scale 1 reproduces the signed codes
    assert np.array_equal(base, O.unpack(packed).astype(np.float32))
    for row in range(3):
        for grp in range(4):
            s = ones.copy()
            s[row, grp] = BF16_HALF
            w = O.dequant(packed, s)
            changed = np.argwhere(w != base)
            assert set(changed[:, 0]) <= {row}
            assert set(changed[:, 1]) <= set(range(32 * grp, 32 * grp + 32))
            assert np.array_equal(w[row, 32 * grp:32 * grp + 32], base[row, 32 * grp:32 * grp + 32] * 0.5)


def test_transpose_free_dx_is_dy_times_w():
    rng = np.random.default_rng(7)
    n, k, m = 48, 96, 5
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = W.f32_to_bf16_bits(rng.uniform(0.01, 0.07, size=(n, k // 32)).astype(np.float32))
    dy = rng.standard_normal((m, n))
    dense = O.dequant(packed, scales).astype(np.float64)
    np.testing.assert_allclose(O.transpose_free_dx(dy, packed, scales), dy @ dense, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ MXFP4 codec


def test_e2m1_table_against_the_fp16_bit_layout():
    # An E2M1 nibble (sign, two exponent bits with bias 1, one mantissa bit) placed
    # into an fp16 word as sign bit 15 and exponent/mantissa bits 11..9 is the same
    # number times 2^-14: fp16 has bias 15 and its own subnormals.  numpy's fp16
    # decoder is independent of the oracle's closed form.
    table = O.e2m1_table()
    bits = np.array([((c & 8) << 12) | ((c & 7) << 9) for c in range(16)], dtype=np.uint16)
    assert np.array_equal(table, bits.view(np.float16).astype(np.float64) * 2.0 ** 14)
    # and the format's known facts: largest magnitude 6, smallest nonzero 0.5, symmetric
    assert table[7] == 6.0 and table[1] == 0.5 and table[0] == 0.0
    assert np.all(np.diff(table[:8]) > 0) and np.array_equal(table[8:], -table[:8])


def test_mxfp4_dequant_nibble_order_and_scale():
    # byte 0x21: low nibble 1 (0.5) first, then 2 (1.0); 0x7F: 15 (-6) then 7 (6);
    # scale 2^-4 (UE8M0 123) and a zero scale (UE8M0 0, bit-cast to +0)
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x21
    packed[0, 1] = 0x7F
    packed[0, 16:] = 0x77
    scales = W.ue8m0_to_bf16_bits(np.array([[123, 0]]))
    assert scales.tolist() == [[BF16_SIXTEENTH, 0]]
    w = O.dequant(packed, scales, "mxfp4")
    assert w[0, :4].tolist() == [0.5 / 16, 1.0 / 16, -6.0 / 16, 6.0 / 16]
    assert np.all(w[0, 4:32] == 0.0) and np.all(w[0, 32:] == 0.0)


def test_ue8m0_bit_cast_is_a_power_of_two():
    e = np.arange(1, 255)
    vals = W.bf16_bits_to_f32(W.ue8m0_to_bf16_bits(e)).astype(np.float64)
    assert np.array_equal(vals, np.array([math.ldexp(1.0, int(k) - 127) for k in e]))


def test_mxfp4_transpose_free_dx_is_dy_times_w():
    rng = np.random.default_rng(8)
    n, k, m = 40, 64, 3
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = W.ue8m0_to_bf16_bits(rng.integers(118, 130, size=(n, k // 32)))
    dy = rng.standard_normal((m, n))
    dense = O.dequant(packed, scales, "mxfp4").astype(np.float64)
    np.testing.assert_allclose(O.transpose_free_dx(dy, packed, scales, "mxfp4"), dy @ dense, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("limit", [0.0, 1.5])
def test_mxfp4_layer_reduces_to_rawint4(limit):
    # An MXFP4 layer whose codes stay within |E2M1| <= 3 is the RAWINT4 layer with
    # code 8 + 2 v and half the scale: the same dense weights, so the oracle must
    # give identical forward and backward results in both formats.
    cfg = W.LayerConfig("m", 3, 2, 64, 96, 4, 8.0, 7, limit, x_std=2.0)
    rng = np.random.default_rng(11)
    table = O.e2m1_table()
    small = np.flatnonzero(np.abs(table) <= 3)  # nibbles 0..5 and 8..13
    w = W.make_weights(cfg, 3)
    mx = W.Weights(gate_packed=w.gate_packed, up_packed=w.up_packed, down_packed=w.down_packed,
                   gate_scale=w.gate_scale, up_scale=w.up_scale, down_scale=w.down_scale, lora=w.lora)
    ri = W.Weights(gate_packed=w.gate_packed, up_packed=w.up_packed, down_packed=w.down_packed,
                   gate_scale=w.gate_scale, up_scale=w.up_scale, down_scale=w.down_scale, lora=w.lora)
    for name in ("gate", "up", "down"):
        shape = getattr(w, name + "_packed").shape
        lo = rng.choice(small, size=shape)
        hi = rng.choice(small, size=shape)
        setattr(mx, name + "_packed", (lo | (hi << 4)).astype(np.uint8))
        to_int = {int(c): int(8 + 2 * table[c]) for c in small}
        lo_i = np.vectorize(to_int.get)(lo)
        hi_i = np.vectorize(to_int.get)(hi)
        setattr(ri, name + "_packed", (lo_i | (hi_i << 4)).astype(np.uint8))
        e = rng.integers(120, 126, size=getattr(w, name + "_scale").shape)
        setattr(mx, name + "_scale", W.ue8m0_to_bf16_bits(e))
        setattr(ri, name + "_scale", W.ue8m0_to_bf16_bits(e - 1))
    batch = W.make_batch(cfg, 5)
    cfg_mx = W.LayerConfig("m", 3, 2, 64, 96, 4, 8.0, 7, limit, x_std=2.0, weight_format="mxfp4")
    a = O.moe(cfg_mx, mx, batch.inputs, batch.expert_ids, batch.route_weights, batch.grad_output)
    b = O.moe(cfg, ri, batch.inputs, batch.expert_ids, batch.route_weights, batch.grad_output)
    assert np.count_nonzero(a["out"]) and np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["dx"], b["dx"]) and np.array_equal(a["droute"], b["droute"])
    for n in O.LORA_NAMES:
        assert np.array_equal(a["grads"][n], b["grads"][n]), n
    # and the full nibble range differs from any RAWINT4 reading
    full = W.make_weights(cfg_mx, 3)
    assert not np.array_equal(O.dequant(full.gate_packed[0], full.gate_scale[0], "mxfp4"),
                              O.dequant(full.gate_packed[0], full.gate_scale[0]))


# ------------------------------------------------------------------ grouping


@pytest.mark.parametrize("index", range(len(W.CONFIGS)))
def test_grouping_against_stable_argsort(index):
    cfg = W.CONFIGS[index]
    ids, _ = W.make_routing(cfg, W.config_seed(index))
    counts, offsets, sorted_slot, bad = O.group(ids, cfg.num_experts)
    flat = ids.ravel()
    assert bad == 0
    assert np.array_equal(counts, np.bincount(flat, minlength=cfg.num_experts))
    assert np.array_equal(offsets[1:], np.cumsum(np.bincount(flat, minlength=cfg.num_experts)))
    assert np.array_equal(sorted_slot, np.argsort(flat, kind="stable"))


def test_grouping_drops_invalid_ids():
    ids = np.array([[3, -1], [0, 4], [3, 0], [9, 3]], dtype=np.int64)
    counts, offsets, sorted_slot, bad = O.group(ids, 4)
    assert bad == 3
    assert counts.tolist() == [2, 0, 0, 3]
    assert offsets.tolist() == [0, 2, 2, 2, 5]
    assert sorted_slot.tolist() == [2, 5, 0, 4, 7]


# ------------------------------------------------------------------ layer helpers


def _uniform_weights(cfg, byte, scale_bits):
    e, h, i = cfg.num_experts, cfg.hidden, cfg.intermediate
    w = W.Weights(
        gate_packed=np.full((e, i, h // 2), byte, dtype=np.uint8),
        up_packed=np.full((e, i, h // 2), byte, dtype=np.uint8),
        down_packed=np.full((e, h, i // 2), byte, dtype=np.uint8),
        gate_scale=np.full((e, i, h // 32), scale_bits, dtype=np.uint16),
        up_scale=np.full((e, i, h // 32), scale_bits, dtype=np.uint16),
        down_scale=np.full((e, h, i // 32), scale_bits, dtype=np.uint16),
    )
    w.lora = {n: np.zeros(s, dtype=np.float32) for n, s in cfg.lora_shapes().items()}
    return w


def _random_case(cfg, seed, x_std=1.0, lora_std=0.05):
    w = W.make_weights(cfg, seed)
    rng = np.random.default_rng(seed)
    for n in w.lora:
        w.lora[n] = (rng.standard_normal(w.lora[n].shape) * lora_std).astype(np.float32)
    x = rng.standard_normal((cfg.qlen, cfg.hidden)) * x_std
    ids = np.stack([rng.permutation(cfg.num_experts)[: cfg.top_k] for _ in range(cfg.qlen)]).astype(np.int64)
    rw = rng.uniform(0.1, 0.9, size=(cfg.qlen, cfg.top_k))
    dy = rng.standard_normal((cfg.qlen, cfg.hidden))
    return w, x, ids, rw, dy


def _run64(cfg, w, x, ids, rw, dy=None, lora=None):
    return O.moe(cfg, w, x, ids, rw, dy, fp32_intermediates=False, inputs_are_bf16=False, lora=lora)


def _dense(w):
    return ([O.dequant(w.gate_packed[e], w.gate_scale[e]).astype(np.float64) for e in range(w.gate_packed.shape[0])],
            [O.dequant(w.up_packed[e], w.up_scale[e]).astype(np.float64) for e in range(w.up_packed.shape[0])],
            [O.dequant(w.down_packed[e], w.down_scale[e]).astype(np.float64) for e in range(w.down_packed.shape[0])])


# ------------------------------------------------------------------ closed forms


@pytest.mark.parametrize("limit", [0.0, 2.0])
def test_hand_case_closed_form(limit):
    # 1 expert, 32 wide: every weight is (9 - 8) * 0.5 = +0.5; B = 0; A_g[0][0] = a
    cfg = _cfg(1, 1, 32, 32, 4, 8.0, 7, limit)  # sc = 2
    w = _uniform_weights(cfg, 0x99, BF16_HALF)
    a = 0.25
    w.lora["gate_lora_a"][0, 0, 0] = a
    vs = [-4.125, -4.0, -3.875, 0.0, 3.875, 4.0, 4.125]
    x = np.zeros((7, 32))
    x[:, 0] = vs
    ids = np.zeros((7, 1), dtype=np.int64)
    rw = np.full((7, 1), 0.75)
    dy = np.ones((7, 32))
    res = _run64(cfg, w, x, ids, rw, dy)
    sc = 2.0
    dbg = np.zeros((32, 4))
    for t, v in enumerate(vs):
        g = u = v / 2
        gp, mg = (min(g, limit), float(g <= limit)) if limit > 0 else (g, 1.0)
        up, mu = (min(max(u, -limit), limit), float(abs(u) <= limit)) if limit > 0 else (u, 1.0)
        y = 16.0 * _silu(gp) * up
        dgv = 12.0 * up * _dsilu(gp) * mg
        duv = 12.0 * _silu(gp) * mu
        np.testing.assert_allclose(res["out"][t], 0.75 * y, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["droute"][t, 0], 32.0 * y, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["dx"][t], 16.0 * (dgv + duv), rtol=1e-12, atol=1e-12)
        dbg[:, 0] += sc * dgv * a * v
    np.testing.assert_allclose(res["grads"]["gate_lora_b"][0], dbg, rtol=1e-12, atol=1e-12)
    for name in ("gate_lora_a", "up_lora_a", "up_lora_b", "down_lora_a", "down_lora_b"):
        assert np.count_nonzero(res["grads"][name]) == 0, name
    if limit == 2.0:
        # worked values: v = 4 sits on the gate bound and passes; v = 4.125 clamps both
        np.testing.assert_allclose(res["out"][5], 0.75 * 16 * 2 * _sig(2.0) * 2, rtol=1e-12)
        assert np.all(res["dx"][6] == 0.0)


def test_supplied_clamp_side_hand_case():
    # the hand case at L = 2 (g = u = v / 2 in every column, B = 0): within the
    # band of a bound the supplied side decides the masks, elsewhere it is ignored
    limit, band = 2.0, 0.1
    cfg = _cfg(1, 1, 32, 32, 4, 8.0, 7, limit)  # sc = 2
    w = _uniform_weights(cfg, 0x99, BF16_HALF)
    a = 0.25
    w.lora["gate_lora_a"][0, 0, 0] = a
    vs = [-4.125, -4.0, -3.875, 0.0, 3.875, 4.0, 4.125]
    x = np.zeros((7, 32))
    x[:, 0] = vs
    ids = np.zeros((7, 1), dtype=np.int64)
    rw = np.full((7, 1), 0.75)
    dy = np.ones((7, 32))
    # v = -4.125: u beyond -L, side inside; v = -4: u on -L, side beyond; v = +-3.875
    # and 0: side = own value, or far from every bound (side ignored); v = 4: g and u on
    # L, side beyond; v = 4.125: both beyond L, side inside
    sides = np.array([-1.99, -2.01, -1.9375, 5.0, 1.9375, 2.01, 1.99])
    side = np.repeat(sides[:, None, None], 32, axis=2)
    res = O.moe(cfg, w, x, ids, rw, dy, fp32_intermediates=False, inputs_are_bf16=False, sides=(side, side),
                band=band, preactivations=True)
    np.testing.assert_array_equal(res["pre_g"][:, 0, :], np.repeat(np.array(vs)[:, None] / 2, 32, axis=1))
    np.testing.assert_array_equal(res["pre_u"], res["pre_g"])
    # masks and clamped values by hand: (gate passes, g', up passes, u')
    decided = {-4.125: (1, -2.0625, 1, -2.0625), -4.0: (1, -2.0, 0, -2.0), -3.875: (1, -1.9375, 1, -1.9375),
               0.0: (1, 0.0, 1, 0.0), 3.875: (1, 1.9375, 1, 1.9375), 4.0: (0, 2.0, 0, 2.0),
               4.125: (1, 2.0625, 1, 2.0625)}
    sc = 2.0
    dbg = np.zeros((32, 4))
    for t, v in enumerate(vs):
        mg, gp, mu, up = decided[v]
        y = 16.0 * _silu(gp) * up
        dgv = 12.0 * up * _dsilu(gp) * mg
        duv = 12.0 * _silu(gp) * mu
        np.testing.assert_allclose(res["out"][t], 0.75 * y, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["droute"][t, 0], 32.0 * y, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["dx"][t], 16.0 * (dgv + duv), rtol=1e-12, atol=1e-12)
        dbg[:, 0] += sc * dgv * a * v
    np.testing.assert_allclose(res["grads"]["gate_lora_b"][0], dbg, rtol=1e-12, atol=1e-12)
    # supplying the oracle's own values changes nothing, to the bit
    plain = O.moe(cfg, w, x, ids, rw, dy, fp32_intermediates=False, inputs_are_bf16=False)
    own = O.moe(cfg, w, x, ids, rw, dy, fp32_intermediates=False, inputs_are_bf16=False,
                sides=(res["pre_g"], res["pre_u"]), band=10.0)
    for key in ("out", "dx", "droute"):
        np.testing.assert_array_equal(own[key], plain[key])
    for n in O.LORA_NAMES:
        np.testing.assert_array_equal(own["grads"][n], plain["grads"][n])


def test_supplied_clamp_side_apriori_band():
    # with the a priori band, an element exactly on a bound (v = 4 at L = 2:
    # g = u = 2) takes the supplied side; one 1/16 away from it (v = 3.875) keeps
    # its own, since its bound is far smaller than that
    limit = 2.0
    cfg = _cfg(1, 1, 32, 32, 4, 8.0, 2, limit)
    w = _uniform_weights(cfg, 0x99, BF16_HALF)
    w.lora["gate_lora_a"][0, 0, 0] = 0.25
    x = np.zeros((2, 32))
    x[:, 0] = [4.0, 3.875]
    ids = np.zeros((2, 1), dtype=np.int64)
    rw = np.full((2, 1), 0.75)
    dy = np.ones((2, 32))
    side = np.repeat(np.array([2.01, 2.01])[:, None, None], 32, axis=2)
    res = O.moe(cfg, w, x, ids, rw, dy, fp32_intermediates=False, inputs_are_bf16=False, sides=(side, side),
                band=O.APRIORI, preactivations=True)
    assert np.all(res["bound_g"] > 0) and np.all(res["bound_g"][1] < 1e-3)
    own = O.moe(cfg, w, x, ids, rw, dy, fp32_intermediates=False, inputs_are_bf16=False)
    # token 0 on the bound: the side beyond L clamps both (no gradient); token 1 unchanged
    assert np.all(res["dx"][0] == 0.0) and np.any(own["dx"][0] != 0.0)
    np.testing.assert_array_equal(res["dx"][1], own["dx"][1])
    np.testing.assert_array_equal(res["out"][1], own["out"][1])


def _fp32_preactivation(wrow, x, A, B, sc, rng):
    """One gate/up pre-activation computed in fp32 by a random summation order, with
    the LoRA factors perturbed by up to 2^-14 (A) and 2^-13 (B, a) relative."""
    prods = (wrow.astype(np.float64) * x).astype(np.float32)  # exact: 11 x 8 significant bits
    acc = np.float32(0.0)
    for k in rng.permutation(prods.size):
        acc = np.float32(acc + prods[k])
    a = np.zeros(A.shape[0], dtype=np.float32)
    for q in range(A.shape[0]):
        ap = (A[q] * (1 + rng.uniform(-2**-14, 2**-14, A.shape[1]))).astype(np.float64)
        t = (ap * x).astype(np.float32)
        s = np.float32(0.0)
        for k in rng.permutation(t.size):
            s = np.float32(s + t[k])
        a[q] = s
    lora = np.float32(0.0)
    for q in rng.permutation(A.shape[0]):
        bq = B[q] * (1 + rng.uniform(-2**-13, 2**-13))
        aq = np.float64(a[q]) * (1 + rng.uniform(-2**-13, 2**-13))
        lora = np.float32(lora + np.float32(sc * bq * aq))
    return np.float32(acc + lora)


@pytest.mark.parametrize("hidden", [256, 7168])
def test_apriori_bound_covers_fp32_computations(hidden):
    # the oracle's a priori bound on a pre-activation's fp32 error covers fp32
    # computations of it in random summation orders with perturbed LoRA factors
    cfg = _cfg(1, 1, hidden, 32, 8, 16.0, 2, 0.0)
    w, x, ids, rw, _ = _random_case(cfg, 41, x_std=2.0, lora_std=0.05)
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)
    ids[:] = 0
    res = O.moe(cfg, w, x, ids, rw, None, inputs_are_bf16=False, preactivations=True)
    wg = O.dequant(w.gate_packed[0], w.gate_scale[0])
    A, B = w.lora["gate_lora_a"][0].astype(np.float64), w.lora["gate_lora_b"][0].astype(np.float64)
    sc = cfg.alpha / cfg.rank
    rng = np.random.default_rng(7)
    worst = 0.0
    for t in range(cfg.qlen):
        for n in range(0, cfg.intermediate, 4):
            g32 = _fp32_preactivation(wg[n], x[t], A, B[n], sc, rng)
            dev = abs(float(g32) - res["pre_g"][t, 0, n])
            bound = res["bound_g"][t, 0, n]
            assert dev <= bound, (t, n, dev, bound)
            worst = max(worst, dev / bound)
    print(f"largest deviation / bound: {worst:.3f}")


def test_duplicate_ids_match_autograd():
    # the routed loop visits every slot: the same expert twice in one token counts twice
    for limit in (0.0, 1.0):
        cfg = _cfg(3, 3, 64, 96, 4, 12.0, 5, limit)
        w, x, ids, rw, dy = _random_case(cfg, 61 + int(limit), x_std=0.5)
        ids[0] = [1, 1, 2]
        ids[1] = [0, 0, 0]
        ids[3] = [2, 0, 2]
        res = _run64(cfg, w, x, ids, rw, dy)
        out, dx, drw, grads = _autograd(cfg, w, x, ids, rw, dy)
        np.testing.assert_allclose(res["out"], out, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(res["dx"], dx, rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(res["droute"], drw, rtol=1e-10, atol=1e-11)
        for n in O.LORA_NAMES:
            np.testing.assert_allclose(res["grads"][n], grads[n], rtol=1e-10, atol=1e-11, err_msg=n)
        # a doubled slot with its route weights summed gives the single slot's output
        ids2, rw2 = ids.copy(), rw.copy()
        ids2[1] = [0, 1, 2]
        rw2[1] = [rw[1].sum(), 0.0, 0.0]
        one = _run64(cfg, w, x, ids2, rw2)
        np.testing.assert_allclose(res["out"][1], one["out"][1], rtol=1e-12, atol=1e-12)


def _page_clamp_case(golden, fp32):
    rows = golden("clamp_example.txt")
    cfg = _cfg(4, 2, 256, 256, 8, 16.0, 9, 2.0)
    w = W.make_weights(cfg, W.BASE_SEED)
    w.gate_packed[:] = 0x99
    w.up_packed[:] = 0x99
    w.up_packed[:, :, 1::2] = 0x77
    w.gate_scale[:] = BF16_HALF
    w.up_scale[:] = BF16_HALF
    for name in ("gate_lora_b", "up_lora_b", "down_lora_b"):
        w.lora[name][:] = 0.0
    x = np.zeros((9, 256))
    for t, x0, x1, _, _ in rows:
        x[int(t), 0] = float(x0)
        x[int(t), 1] = float(x1)
    ids = np.array([[0, 1] if t % 2 == 0 else [1, 0] for t in range(9)], dtype=np.int64)
    rw = np.stack([np.linspace(0.55, 0.75, 9), np.linspace(0.45, 0.25, 9)], axis=1).astype(np.float32)
    dy = W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.random.default_rng(8101).standard_normal((9, 256)) * 0.1))
    res = O.moe(cfg, w, x, ids, rw.astype(np.float64), dy.astype(np.float64), fp32_intermediates=fp32,
                inputs_are_bf16=False)
    return rows, cfg, w, x, ids, rw.astype(np.float64), dy.astype(np.float64), res


@pytest.mark.parametrize("fp32", [False, True])
def test_page_clamp_boundaries(golden, fp32):
    rows, cfg, w, x, ids, rw, dy, res = _page_clamp_case(golden, fp32)
    _, _, wd = _dense(w)
    wu_pattern = np.where((np.arange(256) % 4) < 2, 0.5, -0.5)
    limit = 2.0
    for t, x0, x1, mgate, mup in rows:
        t = int(t)
        g = u = 0.5 * (float(x0) + float(x1))
        assert float(g <= limit) == float(mgate) and float(abs(u) <= limit) == float(mup)
        gp, up = min(g, limit), min(max(u, -limit), limit)
        hv = _silu(gp) * up
        out = np.zeros(256)
        dx = np.zeros(256)
        for s in range(2):
            e = ids[t, s]
            out += rw[t, s] * hv * wd[e].sum(axis=1)
            dh = wd[e].T @ (rw[t, s] * dy[t])
            dgv = dh * up * _dsilu(gp) * float(mgate)
            duv = dh * _silu(gp) * float(mup)
            dx += 0.5 * dgv.sum() + wu_pattern * duv.sum()
        tol = 1e-6 if fp32 else 1e-11
        np.testing.assert_allclose(res["out"][t], out, rtol=tol, atol=tol * np.abs(out).max())
        np.testing.assert_allclose(res["dx"][t], dx, rtol=tol, atol=tol * max(np.abs(dx).max(), 1e-30))
    # tokens 6 and 7 clamp both projections: no gradient reaches their inputs,
    # token 7 only because the decision is made on the fp32 value 2.001953125
    assert np.all(res["dx"][6] == 0.0) and np.all(res["dx"][7] == 0.0)
    assert int(W.f32_to_bf16_bits(np.array([2.001953125], np.float32))[0]) == 0x4000  # rounds onto the bound in bf16
    # tokens 0 and 8 pass only the gate gradient: constant across input columns
    assert np.ptp(res["dx"][0]) <= 1e-6 * np.abs(res["dx"][0]).max()
    assert np.ptp(res["dx"][8]) <= 1e-6 * np.abs(res["dx"][8]).max()


# ------------------------------------------------------------------ textbook and autograd


def _torch_routed(cfg, dense, lora, x, ids, rw):
    """The routed equation in torch ops (float64), token by token, slot by slot."""
    wg, wu, wd = dense
    sc = cfg.alpha / cfg.rank
    limit = cfg.swiglu_limit
    rows = []
    for t in range(x.shape[0]):
        acc = None
        for s in range(ids.shape[1]):
            e = int(ids[t, s])
            xt = x[t:t + 1]
            g = F.linear(xt, wg[e]) + sc * F.linear(F.linear(xt, lora["gate_lora_a"][e]), lora["gate_lora_b"][e])
            u = F.linear(xt, wu[e]) + sc * F.linear(F.linear(xt, lora["up_lora_a"][e]), lora["up_lora_b"][e])
            if limit > 0:
                g = torch.where(g <= limit, g, torch.full_like(g, limit))
                u = torch.where(u < -limit, torch.full_like(u, -limit), torch.where(u > limit, torch.full_like(u, limit), u))
            hh = F.silu(g) * u
            y = F.linear(hh, wd[e]) + sc * F.linear(F.linear(hh, lora["down_lora_a"][e]), lora["down_lora_b"][e])
            term = y * rw[t, s]
            acc = term if acc is None else acc + term
        rows.append(acc)
    return torch.cat(rows, dim=0)


def _autograd(cfg, w, x, ids, rw, dy):
    dense = [[torch.tensor(m) for m in mats] for mats in _dense(w)]
    xt = torch.tensor(x, requires_grad=True)
    rwt = torch.tensor(rw, requires_grad=True)
    lora = {n: torch.tensor(w.lora[n].astype(np.float64), requires_grad=True) for n in O.LORA_NAMES}
    out = _torch_routed(cfg, dense, lora, xt, ids, rwt)
    grads = torch.autograd.grad(out, [xt, rwt] + [lora[n] for n in O.LORA_NAMES], grad_outputs=torch.tensor(dy))
    return out.detach().numpy(), grads[0].numpy(), grads[1].numpy(), {n: g.numpy() for n, g in zip(O.LORA_NAMES, grads[2:])}


def test_textbook_swiglu_mlp():
    # E=1, k=1, rw=1, B=0, no clamp: a plain SwiGLU MLP W_d (silu(W_g x) * W_u x)
    cfg = _cfg(1, 1, 64, 96, 4, 8.0, 5, 0.0)
    w, x, _, _, dy = _random_case(cfg, 11)
    for n in ("gate_lora_b", "up_lora_b", "down_lora_b"):
        w.lora[n][:] = 0.0
    ids = np.zeros((5, 1), dtype=np.int64)
    rw = np.ones((5, 1))
    res = _run64(cfg, w, x, ids, rw, dy)
    wg, wu, wd = (torch.tensor(m[0]) for m in _dense(w))
    xt = torch.tensor(x, requires_grad=True)
    ref = F.linear(F.silu(F.linear(xt, wg)) * F.linear(xt, wu), wd)
    (dx,) = torch.autograd.grad(ref, [xt], grad_outputs=torch.tensor(dy))
    np.testing.assert_allclose(res["out"], ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["dx"], dx.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(res["droute"][:, 0], (ref.detach().numpy() * dy).sum(1), rtol=1e-11)


@pytest.mark.parametrize("limit", [0.0, 1.0])
def test_backward_matches_autograd(limit):
    cfg = _cfg(3, 2, 64, 96, 4, 12.0, 6, limit)
    w, x, ids, rw, dy = _random_case(cfg, 21 + int(limit), x_std=0.5)
    res = _run64(cfg, w, x, ids, rw, dy)
    out, dx, drw, grads = _autograd(cfg, w, x, ids, rw, dy)
    np.testing.assert_allclose(res["out"], out, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(res["dx"], dx, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(res["droute"], drw, rtol=1e-10, atol=1e-11)
    for n in O.LORA_NAMES:
        np.testing.assert_allclose(res["grads"][n], grads[n], rtol=1e-10, atol=1e-11, err_msg=n)
    if limit > 0:
        # the clamp engaged on both sides in this draw
        dense = _dense(w)
        g = np.array([[dense[0][ids[t, s]] @ x[t] for s in range(2)] for t in range(6)])
        assert (g > limit).any() and (g < -limit).any()


def test_merged_weight_identity():
    # LoRA forward equals the base forward with W + sc * B A (dense, fp64)
    cfg = _cfg(2, 2, 64, 64, 8, 4.0, 4, 0.0)
    w, x, ids, rw, _ = _random_case(cfg, 31)
    res = _run64(cfg, w, x, ids, rw)
    sc = cfg.alpha / cfg.rank
    wg, wu, wd = _dense(w)
    L = w.lora
    out = np.zeros_like(x)
    for t in range(cfg.qlen):
        for s in range(cfg.top_k):
            e = ids[t, s]
            mg = wg[e] + sc * L["gate_lora_b"][e].astype(np.float64) @ L["gate_lora_a"][e].astype(np.float64)
            mu = wu[e] + sc * L["up_lora_b"][e].astype(np.float64) @ L["up_lora_a"][e].astype(np.float64)
            md = wd[e] + sc * L["down_lora_b"][e].astype(np.float64) @ L["down_lora_a"][e].astype(np.float64)
            gv, uv = mg @ x[t], mu @ x[t]
            out[t] += rw[t, s] * (md @ (gv / (1 + np.exp(-gv)) * uv))
    np.testing.assert_allclose(res["out"], out, rtol=1e-11, atol=1e-11)


def test_finite_differences():
    cfg = _cfg(2, 2, 32, 32, 4, 8.0, 3, 1.5)
    w, x, ids, rw, dy = _random_case(cfg, 41, x_std=0.6, lora_std=0.2)
    res = _run64(cfg, w, x, ids, rw, dy)
    rng = np.random.default_rng(42)

    def loss(xx=x, rr=rw, lora=None):
        return float((_run64(cfg, w, xx, ids, rr, lora=lora)["out"] * dy).sum())

    def check(analytic, f, eps=1e-6):
        lp, lm, l0 = f(eps), f(-eps), f(0.0)
        fwd, bwd = (lp - l0) / eps, (l0 - lm) / eps
        if abs(fwd - bwd) > 1e-3 * max(1.0, abs(fwd)):
            return False  # a clamp kink lies within the step
        assert abs((lp - lm) / (2 * eps) - analytic) <= 1e-6 * max(1.0, abs(analytic))
        return True

    checked = 0
    for _ in range(10):
        t, c = rng.integers(cfg.qlen), rng.integers(cfg.hidden)

        def fx(d, t=t, c=c):
            xx = x.copy()
            xx[t, c] += d
            return loss(xx=xx)

        checked += check(res["dx"][t, c], fx)
    for t in range(cfg.qlen):
        for s in range(cfg.top_k):
            def fr(d, t=t, s=s):
                rr = rw.copy()
                rr[t, s] += d
                return loss(rr=rr)

            checked += check(res["droute"][t, s], fr)
    for name in O.LORA_NAMES:
        for _ in range(4):
            idx = tuple(rng.integers(0, n) for n in w.lora[name].shape)
            if np.all(ids != idx[0]):
                continue

            def fl(d, name=name, idx=idx):
                lora = {n: w.lora[n].astype(np.float64) for n in O.LORA_NAMES}
                lora[name][idx] += d
                return loss(lora=lora)

            checked += check(res["grads"][name][idx], fl)
    assert checked >= 25


# ------------------------------------------------------------------ invariants


def test_invariants_linearity_permutation_and_windows():
    cfg = _cfg(4, 2, 64, 64, 4, 8.0, 8, 1.0)
    w, x, ids, rw, dy = _random_case(cfg, 51, x_std=0.7)
    base = _run64(cfg, w, x, ids, rw, dy)
    twice = _run64(cfg, w, x, ids, 2 * rw, dy)
    np.testing.assert_allclose(twice["out"], 2 * base["out"], rtol=1e-12)
    np.testing.assert_allclose(twice["dx"], 2 * base["dx"], rtol=1e-12)
    for n in O.LORA_NAMES:
        np.testing.assert_allclose(twice["grads"][n], 2 * base["grads"][n], rtol=1e-12, atol=1e-15)
    perm = np.random.default_rng(3).permutation(cfg.qlen)
    p = _run64(cfg, w, x[perm], ids[perm], rw[perm], dy[perm])
    for key in ("out", "dx", "droute"):
        np.testing.assert_allclose(p[key], base[key][perm], rtol=1e-12, atol=1e-13)
    for n in O.LORA_NAMES:
        np.testing.assert_allclose(p["grads"][n], base["grads"][n], rtol=1e-11, atol=1e-14)
    # window: gradients are sums over tokens, so two half batches add up
    a = _run64(cfg, w, x[:3], ids[:3], rw[:3], dy[:3])
    b = _run64(cfg, w, x[3:], ids[3:], rw[3:], dy[3:])
    sentinel = {n: np.full(s, 7.0) for n, s in cfg.lora_shapes().items()}
    for n in O.LORA_NAMES:
        g = O.finalize_window(sentinel[n], a["grads"][n], accumulate=False, grad_scale=0.5)
        g = O.finalize_window(g, b["grads"][n], accumulate=True, grad_scale=0.5)
        np.testing.assert_allclose(g, 0.5 * base["grads"][n], rtol=1e-11, atol=1e-14)
        inactive = sorted(set(range(cfg.num_experts)) - set(ids[:3].ravel()))
        first = O.finalize_window(sentinel[n], a["grads"][n], accumulate=False, grad_scale=0.5)
        assert all(np.count_nonzero(first[e]) == 0 for e in inactive)


def test_dropped_ids_contribute_nothing():
    cfg = _cfg(4, 2, 64, 64, 4, 8.0, 6, 0.0)
    w, x, ids, rw, dy = _random_case(cfg, 61)
    dropped = ids.copy()
    dropped[1, 0] = -1
    dropped[4, 1] = cfg.num_experts
    zeroed = rw.copy()
    zeroed[1, 0] = 0.0
    zeroed[4, 1] = 0.0
    a = _run64(cfg, w, x, dropped, rw, dy)
    b = _run64(cfg, w, x, ids, zeroed, dy)
    for key in ("out", "dx"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-13)
    for n in O.LORA_NAMES:
        np.testing.assert_allclose(a["grads"][n], b["grads"][n], rtol=1e-12, atol=1e-14)
    assert a["droute"][1, 0] == 0.0 and a["droute"][4, 1] == 0.0


def test_fp32_mode_close_to_fp64_and_deterministic():
    cfg, w, b = W.make_workload(1)
    r32 = O.moe(cfg, w, b.inputs, b.expert_ids, b.route_weights, b.grad_output)
    again = O.moe(cfg, w, b.inputs, b.expert_ids, b.route_weights, b.grad_output)
    r64 = O.moe(cfg, w, b.inputs, b.expert_ids, b.route_weights, b.grad_output, fp32_intermediates=False)
    for key in ("out", "dx", "droute"):
        assert np.array_equal(r32[key], again[key])
        rel, cos = O.relative_l2_and_cosine(r32[key], r64[key])
        assert rel < 1e-4 and cos > 0.99999, key
    for n in O.LORA_NAMES:
        assert np.array_equal(r32["grads"][n], again["grads"][n])
        rel, _ = O.relative_l2_and_cosine(r32["grads"][n], r64["grads"][n])
        assert rel < 1e-4, n


# ------------------------------------------------------------------ metric and frozen base


def test_relative_l2_and_cosine():
    e = np.array([3.0, 4.0])
    assert O.relative_l2_and_cosine(e, e) == (0.0, 1.0)
    rel, cos = O.relative_l2_and_cosine(np.array([3.0, 4.5]), e)
    assert rel == pytest.approx(0.1) and cos == pytest.approx(27.0 / (5.0 * math.hypot(3.0, 4.5)))
    assert O.relative_l2_and_cosine(np.zeros(2), np.zeros(2)) == (0.0, 0.0)


def test_storage_hash_and_frozen_base():
    cfg, w, b = W.make_workload(0)
    before = O.base_storage_hash(w)
    O.moe(cfg, w, b.inputs, b.expert_ids, b.route_weights, b.grad_output)
    assert O.base_storage_hash(w) == before
    # the length prefix separates tensors: [ab] and [a, b] hash differently
    a, bb = np.arange(4, dtype=np.uint8), np.arange(4, 8, dtype=np.uint8)
    assert O.tensor_storage_hash([a, bb]) != O.tensor_storage_hash([np.concatenate([a, bb])])
    w.down_scale[3, -1, -1] ^= 1
    assert O.base_storage_hash(w) != before
