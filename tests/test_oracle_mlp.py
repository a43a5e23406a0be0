"""Pins of the routed-expert MLP oracle (oracle.expert_mlp, bf16_round,
bf16_round_up_abs, expert_mlp_tolerance), against things other than the
oracle itself: exact rational arithmetic for the bf16 rounding, a pure
Python evaluation of the MLP's definition on tiny experts, closed forms
worked out by hand, and brute-force perturbations for the tolerance.
Planted mistakes in MLP variants must fail at least one pin.  CPU only.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from weight_only_block_amd import synth


# ---------------------------------------------------------------- bf16

def _bf16_value(bits: int) -> Fraction:
    b = bits & 0xFFFF
    sign = -1 if b & 0x8000 else 1
    expo = (b >> 7) & 0xFF
    frac = b & 0x7F
    assert expo != 0xFF
    if expo == 0:
        return sign * Fraction(frac) * Fraction(1, 2 ** 133)
    return sign * Fraction(128 + frac) * (Fraction(2) ** (expo - 134))


def _nearest_bf16_brute(v: float) -> int:
    """Round-to-nearest-even by comparing exact rational distances.  bf16
    patterns of one sign are ordered like their magnitudes and the value
    truncated to 16 bits (t) lies within one bf16 step of v, so the
    nearest pattern is among t-2 .. t+2 (all of them are compared)."""
    fv = Fraction(v)
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    t = int(np.array([abs(v)], np.float32).view(np.uint32)[0] >> 16)
    best, best_d = None, None
    for mag in range(max(0, t - 2), min(0x7F7F, t + 2) + 1):
        d = abs(_bf16_value(sign | mag) - fv)
        if best_d is None or d < best_d or (d == best_d and (mag & 1) == 0):
            best, best_d = sign | mag, d
    return best


def test_bf16_round_matches_exact_nearest_even():
    rng = np.random.default_rng(80)
    vals = list(rng.normal(0, 1, 60) * 2.0 ** rng.integers(-140, 120, 60))
    # ties: halfway between neighbours, both parities
    vals += [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 682.5, 2 ** -133 * 1.5, 2 ** -133 * 2.5,
             0.0, -0.0, 2 ** -126 * (1 - 2 ** -9)]
    got = oracle.bf16_round(np.array(vals))
    for v, b in zip(vals, got):
        assert int(b) == _nearest_bf16_brute(float(v)), (v, hex(int(b)))


def test_bf16_round_overflow_and_special_values():
    top = float(_bf16_value(0x7F7F))                 # largest finite bf16
    half_ulp = 2.0 ** 127 * 2 ** -8
    got = oracle.bf16_round(np.array([top, top + half_ulp * 0.99, top + half_ulp, -top - half_ulp,
                                      np.inf, -np.inf, np.nan]))
    assert [int(b) for b in got] == [0x7F7F, 0x7F7F, 0x7F80, 0xFF80, 0x7F80, 0xFF80, 0x7FC0]


def test_bf16_round_up_abs_is_the_next_bf16_at_or_above():
    rng = np.random.default_rng(81)
    vals = np.concatenate([np.abs(rng.normal(0, 1, 300)) * 2.0 ** rng.integers(-140, 100, 300),
                           [0.0, 1.0, 1 + 2 ** -30, 2 ** -133, 2 ** -140]])
    for v, b in zip(vals, oracle.bf16_round_up_abs(vals)):
        b = int(b)
        assert _bf16_value(b) >= Fraction(float(v))
        if b > 0:
            assert _bf16_value(b - 1) < Fraction(float(v))


# -------------------------------------------------------- MLP, definition

def _dequant(codes, scale, minv):
    """The Q4G32 weight w[n][k] = code * scale + min of its 32-group, with
    the even k in the low nibble, read out element by element."""
    N, half = codes.shape
    K = 2 * half
    s = scale.view(np.float16).astype(np.float64)
    m = minv.view(np.float16).astype(np.float64)
    W = [[0.0] * K for _ in range(N)]
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            c = byte & 15 if k % 2 == 0 else byte >> 4
            W[n][k] = c * s[n, k // 32] + m[n, k // 32]
    return W


def _mlp_python(gate, up, down, ids, xs):
    """The MLP's definition in plain Python floats (fp64)."""
    Wg = {e: _dequant(*gate[e]) for e in set(ids)}
    Wu = {e: _dequant(*up[e]) for e in set(ids)}
    Wd = {e: _dequant(*down[e]) for e in set(ids)}
    acts, ys = [], []
    for j, e in enumerate(ids):
        x = [float(v) for v in oracle.bf16_to_f64(xs[j])]
        g = [sum(w * xv for w, xv in zip(row, x)) for row in Wg[e]]
        u = [sum(w * xv for w, xv in zip(row, x)) for row in Wu[e]]
        act = [gi / (1.0 + math.exp(-gi)) * ui if gi >= 0 else gi * math.exp(gi) / (1.0 + math.exp(gi)) * ui
               for gi, ui in zip(g, u)]
        a = [float(_bf16_value(_nearest_bf16_brute(v))) for v in act]
        acts.append(act)
        ys.append([sum(w * av for w, av in zip(row, a)) for row in Wd[e]])
    return np.array(acts), np.array(ys)


def _tiny_experts(seed, n_experts=3, hidden=64, inter=32):
    gate = [synth.q4g32_weights(synth.rng_for(82, seed, 0, e), inter, hidden) for e in range(n_experts)]
    up = [synth.q4g32_weights(synth.rng_for(82, seed, 1, e), inter, hidden) for e in range(n_experts)]
    down = [synth.q4g32_weights(synth.rng_for(82, seed, 2, e), hidden, inter) for e in range(n_experts)]
    return gate, up, down


# Pins written against an MLP implementation mlp(gate, up, down, ids, xs)
# -> (act, act_bits, y), so that planted mistakes can be run through them.

def _oracle_mlp(gate, up, down, ids, xs):
    r = oracle.expert_mlp(gate, up, down, ids, xs)
    return r.act, r.act_bits, r.y


def pin_python_definition(mlp):
    gate, up, down = _tiny_experts(0)
    ids = [2, 0, 2]
    xs = synth.activations(synth.rng_for(83, 0), len(ids), 64)
    act, act_bits, y = mlp(gate, up, down, ids, xs)
    act_py, y_py = _mlp_python(gate, up, down, ids, xs)
    return (np.allclose(act, act_py, rtol=1e-12, atol=1e-300)
            and np.array_equal(oracle.bf16_to_f64(act_bits), oracle.bf16_to_f64(oracle.bf16_round(act_py)))
            and np.allclose(y, y_py, rtol=1e-12, atol=1e-12 * np.abs(y_py).max()))


def _constant_expert(rows, cols, scale, minv, codes=None):
    if codes is None:
        codes = np.zeros((rows, cols // 2), np.uint8)
    return (codes, synth.to_fp16_bits(np.full((rows, cols // 32), scale)),
            synth.to_fp16_bits(np.full((rows, cols // 32), minv)))


def pin_closed_form(mlp):
    # x = 1 everywhere (hidden 32), gate weights all 2 and up weights all
    # 1/3 in fp16 (0.333251953125): g = 64, silu(64) = 64 in fp64 (e^-64 is
    # below half an ulp of 1), u = 32 * 0.333251953125 = 10.6640625,
    # act = 682.5, whose bf16 rounding is 684 (quantum 4 between 512 and
    # 1024; 682.5 is 2.5 above 680).  Down row r with codes c and scale 1/4,
    # min -2: y_r = 684 * sum_n (c_rn / 4 - 2).
    hidden, inter = 32, 32
    gate = [_constant_expert(inter, hidden, 0.0, 2.0)]
    up = [_constant_expert(inter, hidden, 0.0, 1.0 / 3.0)]
    rng = np.random.default_rng(84)
    c = rng.integers(0, 16, size=(hidden, inter))
    down = [(synth.pack_nibbles(c), synth.to_fp16_bits(np.full((hidden, 1), 0.25)),
             synth.to_fp16_bits(np.full((hidden, 1), -2.0)))]
    xs = synth.to_bf16_bits(np.ones((2, hidden), np.float32))
    act, act_bits, y = mlp(gate, up, down, [0, 0], xs)
    want_y = 684.0 * (c / 4.0 - 2.0).sum(axis=1)
    return (np.all(act == 682.5) and np.all(oracle.bf16_to_f64(act_bits) == 684.0)
            and np.array_equal(y, np.stack([want_y, want_y])))


def pin_slot_routing(mlp):
    # Slot j must use expert ids[j] in all three projections: two experts
    # whose down projections differ only by a factor 2 (scale and min
    # doubled, exact in fp16), same gate and up.
    gate, up, down = _tiny_experts(1, n_experts=1)
    d0 = down[0]
    d1 = (d0[0], (d0[1].view(np.float16) * 2).view(np.uint16), (d0[2].view(np.float16) * 2).view(np.uint16))
    xs = synth.activations(synth.rng_for(85, 0), 2, 64)
    _, _, y = mlp(gate * 2, up * 2, [d0, d1], [1, 0], xs[[0, 0]])
    return np.array_equal(y[0], 2.0 * y[1]) and np.any(y[1] != 0)


PINS = [pin_python_definition, pin_closed_form, pin_slot_routing]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_mlp_meets_pin(pin):
    assert pin(_oracle_mlp)


def _wrong_mlps():
    def no_rounding(gate, up, down, ids, xs):
        r = oracle.expert_mlp(gate, up, down, ids, xs)
        # down projection of the fp64 act, as if the input were not bf16
        y = np.stack([np.array(_dequant(*down[e])) @ r.act[j] for j, e in enumerate(ids)])
        return r.act, r.act_bits, y

    def gate_up_swapped(gate, up, down, ids, xs):
        r = oracle.expert_mlp(up, gate, down, ids, xs)
        return r.act, r.act_bits, r.y

    def truncating_bf16(gate, up, down, ids, xs):
        r = oracle.expert_mlp(gate, up, down, ids, xs)
        bits = (r.act.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        y, _ = oracle.grouped_q4g32(down, ids, bits)
        return r.act, bits, y

    def first_expert_only(gate, up, down, ids, xs):
        r = oracle.expert_mlp(gate, up, down, [ids[0]] * len(ids), xs)
        return r.act, r.act_bits, r.y

    def silu_on_up(gate, up, down, ids, xs):
        g, _ = oracle.grouped_q4g32(gate, ids, xs)
        u, _ = oracle.grouped_q4g32(up, ids, xs)
        act = g * oracle.silu(u)
        bits = oracle.bf16_round(act)
        y, _ = oracle.grouped_q4g32(down, ids, bits)
        return act, bits, y

    return {"no bf16 rounding": no_rounding, "gate/up swapped": gate_up_swapped,
            "bf16 by truncation": truncating_bf16, "first slot's expert": first_expert_only,
            "silu on up": silu_on_up}


@pytest.mark.parametrize("name", list(_wrong_mlps()))
def test_planted_mlp_mistakes_are_caught(name):
    wrong = _wrong_mlps()[name]
    assert not all(pin(wrong) for pin in PINS), "no pin catches: " + name


# ------------------------------------------------------------ tolerance

def _bf16_within(target, act, tol):
    """The bf16 nearest to target among those within tol of act (the
    activations the act bar admits): round to nearest, then step one bf16
    towards act where that left the interval."""
    bits = oracle.bf16_round(target).astype(np.int32)
    a = oracle.bf16_to_f64(bits.astype(np.uint16))
    out = np.abs(a - act) > tol
    # one step towards act: magnitude down when |a| > |act| on the same side
    step = np.where((a > act) == (a > 0), -1, 1)
    bits = np.where(out, bits + step, bits)
    a = oracle.bf16_to_f64(bits.astype(np.uint16))
    assert np.all(np.abs(a - act) <= tol)
    return a


def test_mlp_tolerance_bounds_worst_case_activations():
    # Move each activation anywhere inside its tolerance (towards the sign
    # of the down weights, against it, and at random), round to bf16 as a
    # kernel would, and add the largest down-GEMV error the bar allows: the
    # result must stay inside tol_y.
    gate, up, down = _tiny_experts(2)
    ids = [0, 1, 2, 1]
    xs = synth.activations(synth.rng_for(86, 0), len(ids), 64)
    ref = oracle.expert_mlp(gate, up, down, ids, xs)
    tol_act, tol_y = oracle.expert_mlp_tolerance(ref, down, ids)
    assert np.all(tol_act > 0) and np.all(tol_y >= 2e-3 * ref.a_y)
    rng = np.random.default_rng(87)
    for j, e in enumerate(ids):
        W = np.array(_dequant(*down[e]))
        for trial in range(6):
            if trial < 2:
                sgn = np.sign(W[trial * 7 % W.shape[0]]) * (1 if trial == 0 else -1)
            else:
                sgn = rng.uniform(-1, 1, W.shape[1])
            a_k = _bf16_within(ref.act[j] + sgn * tol_act[j], ref.act[j], tol_act[j])
            y_exact = W @ a_k
            worst = y_exact + np.sign(y_exact - ref.y[j]) * 2e-3 * (np.abs(W) @ np.abs(a_k))
            assert np.all(np.abs(worst - ref.y[j]) <= tol_y[j] * (1 + 1e-12))
