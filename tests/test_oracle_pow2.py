"""Pins of the oracle's power-of-two scale rule: the variant in which each
group scale is a power of two, so that gfx950's scaled matrix instruction
can apply it through an E8M0 exponent.  The pages recommend that hardware
apply fine-grained group scales inside the matrix instruction
(why-be.why-be.co.kr page, hardware-design passage); E8M0 carries exponents
only, so the scale is rounded up to the next power of two.

Rule: s = 2^e with e the smallest integer such that amax <= 448 * 2^e,
clamped to [-127, 127]; inv = 2^-e; codes = encode(x * inv)."""
import math

import numpy as np
import pytest

from fp8_fine_grained_quant_amd import synth


def _f32(v) -> float:
    return float(np.float32(v))


@pytest.mark.parametrize("seed", range(3))
def test_pow2_scale_closed_form(oracle, seed):
    rng = np.random.default_rng(seed)
    amax = (np.exp(rng.uniform(-80, 80, 4000)) * rng.uniform(0.5, 1.0, 4000)).astype(np.float32)
    for a in amax:
        a = float(a)
        s, inv = oracle.group_scale_pow2(a)
        m, ex = math.frexp(float(s))
        assert m == 0.5, "scale not a power of two"
        e = ex - 1
        if -127 < e < 127:
            assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1), (a, e)
        assert float(inv) == 2.0 ** -e


def test_pow2_scale_edges(oracle):
    assert oracle.group_scale_pow2(0.0) == (np.float32(2.0 ** -127), np.float32(2.0 ** 127))
    assert oracle.group_scale_pow2(1e-40)[0] == np.float32(2.0 ** -127)    # clamped
    for j in range(-100, 100, 7):                                        # exact 448 * 2^j
        s, inv = oracle.group_scale_pow2(_f32(448.0 * 2.0 ** j))
        assert float(s) == 2.0 ** j and float(inv) == 2.0 ** -j
        s, _ = oracle.group_scale_pow2(float(np.nextafter(np.float32(448.0 * 2.0 ** j),
                                                          np.float32(np.inf))))
        assert float(s) == 2.0 ** (j + 1)


def test_pow2_equals_fp32_rule_when_amax_is_448_times_a_power_of_two(oracle):
    """Where every group's amax is 448 * 2^j the two rules give the same
    scale and inverse, so all codes and scales must coincide."""
    rng = np.random.default_rng(5)
    R, C = 64, 512
    x = (rng.standard_normal((R, C)) * 30).astype(np.float32)
    x = np.clip(x, -447.0, 447.0)
    js = rng.integers(-20, 20, (R, C // 128))
    for r in range(R):
        for g in range(C // 128):
            x[r, g * 128 + rng.integers(0, 128)] = 448.0
            x[r, g * 128:(g + 1) * 128] *= np.float32(2.0 ** js[r, g])
    q0, s0 = oracle.quant_1x128(x)
    q1, s1 = oracle.quant_1x128(x, rule=oracle.RULE_POW2)
    assert np.array_equal(q0, q1) and np.array_equal(s0.view(np.uint32), s1.view(np.uint32))


def test_pow2_scaling_invariance(oracle):
    """Scaling a tensor by 2^j leaves the codes unchanged and multiplies
    every scale by 2^j (both exact under the rule)."""
    a = synth.bf16_bits_to_f32(synth.fprop_inputs(256, 256, 1024)[0])
    q, s = oracle.quant_1x128(a, rule=oracle.RULE_POW2)
    for j in (-9, 5, 30):
        qj, sj = oracle.quant_1x128((a * np.float32(2.0 ** j)).astype(np.float32),
                                    rule=oracle.RULE_POW2)
        assert np.array_equal(qj, q)
        assert np.array_equal(sj, (s * np.float32(2.0 ** j)).astype(np.float32))
    w = synth.bf16_bits_to_f32(synth.fprop_inputs(256, 384, 1024)[1])
    qw, sw, qt = oracle.quant_128x128(w, with_transpose=True, rule=oracle.RULE_POW2)
    qw2, sw2, _ = oracle.quant_128x128((w * np.float32(2.0 ** 7)).astype(np.float32),
                                       rule=oracle.RULE_POW2)
    assert np.array_equal(qw, qw2) and np.array_equal(sw2, sw * np.float32(128.0))
    assert np.array_equal(qt, qw.T)


def test_pow2_exactly_representable(oracle):
    """x = decode(b) * 2^e0 with one |b| = 448 per group: s = 2^e0, q = b."""
    rng = np.random.default_rng(8)
    R, C = 32, 640
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    b = rng.choice(finite, size=(R, C)).astype(np.uint8)
    e0 = rng.integers(-30, 30, (R, C // 128))
    for r in range(R):
        for g in range(C // 128):
            b[r, g * 128 + rng.integers(0, 128)] = 0x7E | (0x80 if rng.random() < 0.5 else 0)
    dec = oracle.e4m3_decode(b)
    x = (dec * np.repeat(2.0 ** e0, 128, axis=1)).astype(np.float32)
    q, s = oracle.quant_1x128(x, rule=oracle.RULE_POW2)
    assert np.array_equal(q, b)
    assert np.array_equal(s, (2.0 ** e0.T).astype(np.float32))


def test_pow2_error_bound_and_range_use(oracle):
    """Every group's amax lands in (224, 448] after scaling, and each value
    is within half an E4M3 step of its code (relative 2^-4 in the normal
    range, 2^-10 absolute in scaled units below it)."""
    x = synth.bf16_bits_to_f32(synth.fprop_inputs(512, 256, 2048)[0])
    q, s = oracle.quant_1x128(x, rule=oracle.RULE_POW2)
    sx = x.astype(np.float64) / np.repeat(s.T.astype(np.float64), 128, axis=1)
    amax = np.abs(sx).reshape(512, -1, 128).max(axis=2)
    assert np.all(amax > 224.0) and np.all(amax <= 448.0)
    err = np.abs(oracle.e4m3_decode(q) - sx)
    assert np.all(err <= np.maximum(np.abs(sx) * 2.0 ** -4, 2.0 ** -10) + 1e-12)
