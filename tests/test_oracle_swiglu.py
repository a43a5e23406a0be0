"""Pins for the oracle's SwiGLU step (act = silu(gate) * up) and its
tolerance, against facts that do not come from the oracle's own formula:
hand-worked values, closed forms of the logistic function, the identity
silu(z) - silu(-z) = z, asymptotes, and a randomized check that the stated
error bound really bounds the error.  A planted-mistake test shows each
plausible slip in silu fails at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from weight_only_block_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _codes_from_hex(rows, K):
    return np.array([list(bytes.fromhex(h)) for h in rows], np.uint8).reshape(len(rows), K // 2)


# Pins written against a silu implementation, so the planted-mistake test
# below can run them on wrong variants.

def pin_closed_forms(silu):
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 (hand-derived).
    v = silu(np.array([0.0, math.log(3.0), -math.log(3.0)]))
    return (v[0] == 0.0 and abs(v[1] - 0.75 * math.log(3.0)) < 1e-15
            and abs(v[2] + 0.25 * math.log(3.0)) < 1e-15)


def pin_odd_part(silu):
    # sigmoid(z) + sigmoid(-z) = 1  =>  silu(z) - silu(-z) = z.
    z = np.linspace(-30.0, 30.0, 6001)
    return np.allclose(silu(z) - silu(-z), z, rtol=1e-13, atol=1e-13)


def pin_asymptotes(silu):
    with np.errstate(over="raise", invalid="raise", divide="raise"):
        big = silu(np.array([40.0, 100.0, 800.0]))
        small = silu(np.array([-40.0, -100.0, -800.0]))
    return (np.allclose(big, [40.0, 100.0, 800.0], rtol=1e-15, atol=0)
            and np.all(np.abs(small) <= np.abs([-40.0, -100.0, -800.0]) * np.exp([-40.0, -100.0, -700.0]))
            and np.all(small <= 0.0))


def pin_golden(silu):
    d = json.load(open(os.path.join(GOLDEN, "q4g32_swiglu_two_rows.json")))
    g = np.array(d["gate_out"], np.float64)
    u = np.array(d["up_out"], np.float64)
    return np.allclose(silu(g) * u, d["act"], rtol=1e-14, atol=0)


PINS = [pin_closed_forms, pin_odd_part, pin_asymptotes, pin_golden]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_silu_meets_pin(pin):
    assert pin(oracle.silu)


def _wrong_silus():
    def stable(fn):
        def wrapped(z):
            with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
                return fn(np.asarray(z, np.float64))
        return wrapped
    return {
        "exp sign flipped": stable(lambda z: z / (1.0 + np.exp(z))),
        "sigmoid only": stable(lambda z: 1.0 / (1.0 + np.exp(-z))),
        "base 2": stable(lambda z: z / (1.0 + np.exp2(-z))),
        "tanh in place of sigmoid": stable(lambda z: z * np.tanh(z)),
        "scaled input (gelu-like)": stable(lambda z: z / (1.0 + np.exp(-1.702 * z))),
        "naive overflowing form": lambda z: np.asarray(z, np.float64) * np.exp(z) / (1.0 + np.exp(z)),
    }


@pytest.mark.parametrize("name", list(_wrong_silus()))
def test_planted_silu_mistakes_are_caught(name):
    wrong = _wrong_silus()[name]
    caught = False
    for pin in PINS:
        try:
            ok = pin(wrong)
        except (FloatingPointError, ValueError):
            ok = False
        caught = caught or not ok
    assert caught, "no pin catches: " + name


def test_slope_bound_covers_the_derivative():
    # silu'(z) = s (1 + z (1 - s)), s = sigmoid(z); its maximum is ~1.09984.
    z = np.linspace(-50.0, 50.0, 1_000_001)
    s = 1.0 / (1.0 + np.exp(-z))
    d = s * (1.0 + z * (1.0 - s))
    assert d.max() <= oracle.SILU_SLOPE_BOUND
    assert d.max() >= oracle.SILU_SLOPE_BOUND - 2e-4     # the bound is not loose
    assert d.min() >= -oracle.SILU_SLOPE_BOUND


def test_grouped_swiglu_golden_example():
    d = json.load(open(os.path.join(GOLDEN, "q4g32_swiglu_two_rows.json")))
    K = d["K"]
    gate = (_codes_from_hex(d["gate"]["codes_hex_by_row"], K),
            np.array(d["gate"]["scale_fp16_bits"], np.uint16), np.array(d["gate"]["min_fp16_bits"], np.uint16))
    up = (_codes_from_hex(d["up"]["codes_hex_by_row"], K),
          np.array(d["up"]["scale_fp16_bits"], np.uint16), np.array(d["up"]["min_fp16_bits"], np.uint16))
    for vals, bits in ((d["gate"]["scale_values"], gate[1]), (d["up"]["min_values"], up[2])):
        assert np.array_equal(bits.view(np.float16).astype(np.float64), vals)
    x = np.stack([np.full(K, 0x3F80, np.uint16), np.full(K, 0x4000, np.uint16)])
    act, g, u, _, _ = oracle.grouped_q4g32_swiglu([gate], [up], d["ids"], x)
    assert np.array_equal(g, d["gate_out"]) and np.array_equal(u, d["up_out"])
    assert np.allclose(act, d["act"], rtol=1e-14, atol=0)


def test_swiglu_is_linear_in_up_and_zero_gate_gives_zero():
    rng = synth.rng_for(50, 0)
    N, K = 64, 256
    gate = synth.q4g32_weights(rng, N, K)
    up = synth.q4g32_weights(rng, N, K)
    # Doubling every up scale and min doubles up exactly (fp16 exponent + 1).
    up2 = (up[0], (up[1].view(np.float16) * 2).view(np.uint16), (up[2].view(np.float16) * 2).view(np.uint16))
    x = synth.activations(rng, 3, K)
    a1 = oracle.grouped_q4g32_swiglu([gate], [up], [0, 0, 0], x)[0]
    a2 = oracle.grouped_q4g32_swiglu([gate], [up2], [0, 0, 0], x)[0]
    assert np.array_equal(a2, 2 * a1)
    zero_gate = (gate[0], np.zeros_like(gate[1]), np.zeros_like(gate[2]))
    assert np.all(oracle.grouped_q4g32_swiglu([zero_gate], [up], [0, 0, 0], x)[0] == 0.0)


def test_swiglu_tolerance_bounds_worst_case_perturbations():
    # Perturb g and u anywhere inside the GEMV bar (corners and random
    # points) and check the change of silu(g) u stays within the bound E
    # E (the tolerance before its fp32 and bf16 rounding terms).
    rng = np.random.default_rng(51)
    g = rng.normal(0, 4, 20000)
    u = rng.normal(0, 4, 20000)
    a_g = np.abs(g) + rng.uniform(0, 50, g.size)
    a_u = np.abs(u) + rng.uniform(0, 50, u.size)
    act = oracle.swiglu(g, u)
    E = oracle.swiglu_propagated_bound(g, u, a_g, a_u)
    assert np.all(oracle.swiglu_tolerance(act, g, u, a_g, a_u) >= E)
    dg, du = 2e-3 * a_g, 2e-3 * a_u
    for sg, su in ((1, 1), (1, -1), (-1, 1), (-1, -1), (None, None)):
        if sg is None:
            pg, pu = rng.uniform(-1, 1, g.size), rng.uniform(-1, 1, g.size)
        else:
            pg, pu = sg, su
        moved = oracle.swiglu(g + pg * dg, u + pu * du)
        assert np.all(np.abs(moved - act) <= E * (1 + 1e-12) + 1e-300)


def test_swiglu_tolerance_covers_bf16_rounding_of_exact_values():
    # With exact gate/up sums only the fp32 evaluation and the bf16 rounding
    # remain; round-to-nearest-even to 8 significant bits of any value must
    # stay inside the bound (values just above a power of two are the worst).
    rng = np.random.default_rng(52)
    vals = np.concatenate([2.0 ** rng.integers(-20, 20, 5000) * (1 + rng.uniform(0, 2 ** -7, 5000)),
                           rng.normal(0, 100, 5000)])
    f32 = vals.astype(np.float32).view(np.uint32).astype(np.uint64)
    rounded = ((f32 + 0x7FFF + ((f32 >> 16) & 1)) >> 16) << 16
    bf = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
    zero = np.zeros_like(vals)
    tol = oracle.swiglu_tolerance(vals, zero + 50.0, zero, zero, zero)
    assert np.all(np.abs(bf - vals) <= tol)
