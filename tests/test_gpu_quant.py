"""GPU parity of the quantizers: every code byte and every FP32 scale bit
pattern must equal the CPU oracle's (1x128 activation tiles and 128x128
weight blocks, "Should Fixing Deepseek Take 60 Steps?", Figure 7(a); 128x1
groups along tokens for the weight-gradient GEMM)."""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

from fp8_fine_grained_quant_amd import synth
from helpers import assert_same_bytes, codes, scale_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp8_fine_grained_quant_amd as fq
    return fq


def _check_1x128(fq, oracle, x, transposed=False, what=""):
    q, s = fq.fp8_quant_1x128(to_dev(x), transposed=transposed)
    qo, so = oracle.quant_1x128(x, transposed=transposed)
    torch.cuda.synchronize()
    assert_same_bytes(codes(q), qo, what + " codes")
    assert_same_bytes(scale_bits(s), so.view(np.uint32), what + " scales")


def test_quant_1x128_tiny_f32(fq, oracle):
    a, _ = synth.tiny_inputs()
    _check_1x128(fq, oracle, a, what="A[256,512] f32")


def test_quant_1x128_fprop_activation(fq, oracle):
    a, _ = synth.fprop_inputs(n=128)            # A[8192,7168] bf16 with outliers (W unused)
    _check_1x128(fq, oracle, a, what="A[8192,7168] bf16")


def test_quant_1x128_dgrad_output_grad(fq, oracle):
    dy = synth.f32_to_bf16_bits(synth.normal_f32((8192, 18432), 1e-3, 301))
    _check_1x128(fq, oracle, dy, what="dY[8192,18432] bf16")


def test_quant_128x1_wgrad_operands(fq, oracle):
    dy, x = synth.wgrad_inputs()
    _check_1x128(fq, oracle, dy, transposed=True, what="dY^T 128x1")
    _check_1x128(fq, oracle, x, transposed=True, what="X^T 128x1")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (37, 300), (129, 128), (5, 1000), (260, 136)])
def test_quant_1x128_ragged(fq, oracle, dtype, shape):
    rng = np.random.default_rng(shape[0] * 1000 + shape[1])
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-5, 5, (shape[0], 1)))).astype(np.float32)
    if dtype == "bf16":
        x = synth.f32_to_bf16_bits(x)
    _check_1x128(fq, oracle, x, what=f"{shape} {dtype}")
    _check_1x128(fq, oracle, x, transposed=True, what=f"{shape} {dtype} transposed")


def test_quant_1x128_padded_leading_dims_untouched(fq, oracle):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((40, 384)).astype(np.float32)
    xd = torch.zeros((40, 520), dtype=torch.float32, device="cuda")
    xd[:, :384] = to_dev(x)
    q = torch.full((40, 400), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((3, 48), float("nan"), dtype=torch.float32, device="cuda")
    fq.fp8_quant_1x128(xd[:, :384], q=q[:, :384], s=s[:, :40])
    qo, so = oracle.quant_1x128(x)
    assert_same_bytes(codes(q)[:, :384], qo, "codes")
    assert np.all(codes(q)[:, 384:] == 0xA5), "row padding of q was written"
    assert_same_bytes(scale_bits(s)[:, :40], so.view(np.uint32), "scales")
    assert torch.isnan(s[:, 40:]).all(), "padding of s was written"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_1x128_tile_path_edges(fq, oracle, dtype):
    """Row counts around the switch from the row-striding kernel (fewer than
    128 rows) to 32x128 tiles, ragged last tiles in both directions, and
    inputs and outputs that only allow element accesses: an input view one
    element off its 16-byte alignment, a row pitch that is not a multiple of
    16 bytes, and code rows whose pitch is not a multiple of 8."""
    rng = np.random.default_rng(77 if dtype == "f32" else 78)
    for R, C in [(127, 128), (128, 128), (129, 129), (159, 1000), (160, 256), (161, 385)]:
        x = (rng.standard_normal((R, C)) * np.exp(rng.uniform(-6, 6, (R, 1)))).astype(np.float32)
        if dtype == "bf16":
            x = synth.f32_to_bf16_bits(x)
        _check_1x128(fq, oracle, x, what=f"{R}x{C} {dtype}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    R, C = 200, 300
    x = (rng.standard_normal((R, C)) * np.exp(rng.uniform(-6, 6, (R, 1)))).astype(np.float32)
    xo = to_dev(x).to(tdt)
    xv = xo.float().cpu().numpy()
    qo, so = oracle.quant_1x128(xv)
    # input one element past a 16-byte boundary, row pitch C+3 elements
    buf = torch.zeros((R, C + 3), dtype=tdt, device="cuda")
    buf[:, 1:C + 1] = xo
    q = torch.full((R, C + 5), 0x5A, dtype=torch.uint8, device="cuda")   # code pitch not a multiple of 8
    s = torch.full(((C + 127) // 128, R + 3), float("nan"), dtype=torch.float32, device="cuda")
    fq.fp8_quant_1x128(buf[:, 1:C + 1], q=q[:, :C], s=s[:, :R])
    torch.cuda.synchronize()
    assert_same_bytes(codes(q)[:, :C], qo, f"unaligned {dtype} codes")
    assert np.all(codes(q)[:, C:] == 0x5A), "row padding of q was written"
    assert_same_bytes(scale_bits(s)[:, :R], so.view(np.uint32), f"unaligned {dtype} scales")
    assert torch.isnan(s[:, R:]).all(), "padding of s was written"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_128x1_edges(fq, oracle, dtype):
    """128x1 groups (the transposed view) on ragged 128-row groups and
    ragged 256-column tiles, with an input view one element off its 16-byte
    alignment and padded pitches for the input, the transposed codes (not a
    multiple of 8) and the scales (not a multiple of 4): element accesses
    throughout, and the padding left untouched."""
    rng = np.random.default_rng(91 if dtype == "f32" else 92)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for T, C in [(300, 300), (128, 257), (129, 64)]:
        x = (rng.standard_normal((T, C)) * np.exp(rng.uniform(-6, 6, (1, C)))).astype(np.float32)
        xo = to_dev(x).to(tdt)
        qo, so = oracle.quant_1x128(xo.float().cpu().numpy(), transposed=True)
        buf = torch.zeros((T, C + 3), dtype=tdt, device="cuda")
        buf[:, 1:C + 1] = xo
        g = (T + 127) // 128
        q = torch.full((C, T + 5), 0x5A, dtype=torch.uint8, device="cuda")
        sc = torch.full((g, C + 3), float("nan"), dtype=torch.float32, device="cuda")
        fq.fp8_quant_1x128(buf[:, 1:C + 1], transposed=True, q=q[:, :T], s=sc[:, :C])
        torch.cuda.synchronize()
        what = f"128x1 {T}x{C} {dtype}"
        assert_same_bytes(codes(q)[:, :T], qo, what + " codes")
        assert np.all(codes(q)[:, T:] == 0x5A), what + ": row padding of q was written"
        assert_same_bytes(scale_bits(sc)[:, :C], so.view(np.uint32), what + " scales")
        assert torch.isnan(sc[:, C:]).all(), what + ": padding of s was written"


def test_quant_1x128_special_groups(fq, oracle):
    x = np.zeros((8, 512), dtype=np.float32)
    x[1, :128] = -0.0                                  # all negative zero
    x[2, 128:256] = 1e-40                              # FP32 subnormal amax
    x[2, 130] = -3e-41
    x[3, 256:384] = np.float32(3.0e38)                 # near FLT_MAX
    x[3, 300] = -np.float32(3.4e38)
    x[4, :] = np.float32(448.0)
    x[4, 1::2] = -np.float32(447.99997)
    x[5, :] = np.linspace(-2.0 ** -10, 2.0 ** -10, 512, dtype=np.float32)
    x[6, :] = np.float32(1e-37)                        # 448/amax overflows to +inf -> FLT_MAX
    x[6, 7] = 5e-38
    x[7, :] = np.float32(3.2e-43)                      # amax/448 is the smallest subnormal
    _check_1x128(fq, oracle, x, what="special groups")
    _check_1x128(fq, oracle, np.ascontiguousarray(x[:, :256].T.copy()), transposed=True,
                 what="special groups transposed")


def _check_128x128(fq, oracle, w, with_t, what):
    q, s, qt = fq.fp8_quant_128x128(to_dev(w), with_transpose=with_t)
    qo, so, qto = oracle.quant_128x128(w, with_transpose=with_t)
    torch.cuda.synchronize()
    assert_same_bytes(codes(q), qo, what + " codes")
    assert_same_bytes(scale_bits(s), so.view(np.uint32), what + " scales")
    if with_t:
        assert_same_bytes(codes(qt), qto, what + " transposed codes")


def test_quant_128x128_tiny_f32(fq, oracle):
    _, w = synth.tiny_inputs()
    _check_128x128(fq, oracle, w, True, "W[256,512] f32")


def test_quant_128x128_fprop_weight(fq, oracle):
    w = synth.f32_to_bf16_bits(synth.normal_f32((18432, 7168), 0.02, 202))
    _check_128x128(fq, oracle, w, True, "W[18432,7168] bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1), (7, 3), (300, 200), (128, 136), (257, 1000)])
def test_quant_128x128_ragged(fq, oracle, dtype, shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    w = rng.standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        w = synth.f32_to_bf16_bits(w)
    _check_128x128(fq, oracle, w, True, f"{shape} {dtype}")


def test_quant_repeatable(fq):
    a, _ = synth.fprop_inputs(m=2048, n=128)
    xd = to_dev(a)
    q1, s1 = fq.fp8_quant_1x128(xd)
    q2, s2 = fq.fp8_quant_1x128(xd)
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def _encode_chunk_expected(oracle, bits: np.ndarray) -> np.ndarray:
    parts = np.array_split(bits, 8)
    with cf.ThreadPoolExecutor(8) as ex:
        outs = list(ex.map(lambda b: oracle.e4m3_encode(b.view(np.float32)), parts))
    return np.concatenate(outs)


def test_encode_every_fp32_pattern_up_to_448(fq, oracle):
    """Every FP32 bit pattern with |v| <= 448, through the public quantizer:
    each 1x128 group holds 448 (so inv = 448/448 = 1 and x*inv = x exactly)
    and 127 patterns; their codes must equal the oracle's encoder."""
    top = int(np.array([448.0], np.float32).view(np.uint32)[0])      # 0x43E00000
    chunk = 127 * (1 << 19)
    starts = list(range(0, top + 1, chunk))
    done = 0
    for sign in (0, 0x80000000):
        for st in starts:
            n = min(chunk, top + 1 - st)
            ngroups = (n + 126) // 127
            pat = torch.arange(st, st + n, dtype=torch.int64, device="cuda")
            pat = (pat | sign).to(torch.int64)
            pat32 = (pat - (1 << 32) * (pat >= (1 << 31))).to(torch.int32)
            xs = torch.zeros((ngroups, 128), dtype=torch.float32, device="cuda")
            xs[:, 0] = 448.0
            flat = xs[:, 1:].reshape(-1)
            flat[:n] = pat32.view(torch.float32)
            xs[:, 1:] = flat.view(ngroups, 127)
            q, s = fq.fp8_quant_1x128(xs)
            got = q[:, 1:].reshape(-1)[:n].cpu().numpy()
            assert torch.all(s == 1.0)
            bits = (np.arange(st, st + n, dtype=np.uint64) | sign).astype(np.uint32)
            exp = _encode_chunk_expected(oracle, bits)
            if not np.array_equal(got, exp):
                i = np.flatnonzero(got != exp)[0]
                v = bits[i:i + 1].view(np.float32)[0]
                raise AssertionError(f"pattern {bits[i]:#010x} ({v!r}): gpu {got[i]:#04x} "
                                     f"oracle {exp[i]:#04x}")
            done += n
    assert done == 2 * (top + 1)


# Every positive finite FP32 amax, 0x00000001 .. 0x7F7FFFFF, in 16 parts.
_AMAX_LAST = 0x7F7FFFFF
_AMAX_PARTS = 16


@pytest.mark.parametrize("part", range(_AMAX_PARTS))
def test_scale_division_every_positive_amax(fq, oracle, part):
    """The scale rule s = amax/448, inv = min(448/amax, FLT_MAX) with IEEE
    round-to-nearest divisions and no denormal flush, for every positive
    finite FP32 amax.  Each row [amax, y] is its own group (the row is 2
    wide): s checks the first division bit for bit.  y = fl32(amax * 27/28)
    puts y * inv within a few ulps of 432, the rounding midpoint between the
    E4M3 values 416 and 448, so y's code depends on the last bits of inv and
    checks the second division (and the clamp below amax = 448/FLT_MAX)."""
    span = (_AMAX_LAST + _AMAX_PARTS - 1) // _AMAX_PARTS
    lo = 1 + part * span
    hi = min(_AMAX_LAST + 1, lo + span)
    chunk = 1 << 25
    ratio = np.float32(27.0 / 28.0)
    near_mid = 0
    for a0 in range(lo, hi, chunk):
        a1 = min(hi, a0 + chunk)
        amax = np.arange(a0, a1, dtype=np.uint32).view(np.float32)
        x = np.empty((a1 - a0, 2), dtype=np.float32)
        x[:, 0] = amax
        x[:, 1] = amax * ratio
        q, s = fq.fp8_quant_1x128(torch.from_numpy(x).cuda())
        qo, so = oracle.quant_1x128(x)
        torch.cuda.synchronize()
        sg = s.cpu().numpy().view(np.uint32).reshape(-1)
        bad = np.flatnonzero(sg != so.view(np.uint32).reshape(-1))
        assert bad.size == 0, (f"scale of amax {amax[bad[0]]!r} ({a0 + bad[0]:#010x}): gpu "
                               f"{sg[bad[0]]:#010x} oracle {so.view(np.uint32).reshape(-1)[bad[0]]:#010x}")
        qg = q.cpu().numpy()
        bad = np.flatnonzero((qg != qo).any(axis=1))
        assert bad.size == 0, (f"codes of row {x[bad[0]]!r}: gpu {qg[bad[0]]} oracle {qo[bad[0]]}")
        near_mid += int(np.count_nonzero((qo[:, 1] & 0x7F) == 0x7E))
    # y's code must split between 0x7D (416) and 0x7E (448) across the range:
    # the case is sensitive to inv's rounding, not stuck on one side
    assert 0 < near_mid < hi - lo


def test_quant_random_shapes(fq, oracle):
    """60 seeded random cases, bit for bit against the oracle: shapes up to
    1500 x 1500, BF16 or FP32 input, rows scaled over e^+-8 with 1 % exact
    zeros, FP32 or power-of-two scale rule, and each of the three groupings
    (1x128, 128x1 on the stored tensor, 128x128)."""
    rng = np.random.default_rng(4242)
    for case in range(60):
        R, C = int(rng.integers(1, 1500)), int(rng.integers(1, 1500))
        pow2 = rng.random() < 0.3
        rule = oracle.RULE_POW2 if pow2 else oracle.RULE_FP32
        x = (rng.standard_normal((R, C)) * np.exp(rng.uniform(-8, 8, (R, 1)))).astype(np.float32)
        x[rng.random((R, C)) < 0.01] = 0.0
        bf = rng.random() < 0.7
        xd = to_dev(x).to(torch.bfloat16) if bf else to_dev(x)
        xo = xd.float().cpu().numpy()           # the values the device quantizes (BF16 is exact in FP32)
        kind = int(rng.integers(0, 3))
        if kind == 0:
            q, s = fq.fp8_quant_1x128(xd, pow2=pow2)
            qo, so = oracle.quant_1x128(xo, rule=rule)
        elif kind == 1:
            q, s = fq.fp8_quant_1x128(xd, transposed=True, pow2=pow2)
            qo, so = oracle.quant_1x128(xo, transposed=True, rule=rule)
        else:
            q, s, _ = fq.fp8_quant_128x128(xd, pow2=pow2)
            qo, so, _ = oracle.quant_128x128(xo, rule=rule)
        torch.cuda.synchronize()
        what = f"case {case}: grouping {kind} {R}x{C} {'bf16' if bf else 'f32'} pow2={pow2}"
        assert_same_bytes(codes(q), qo, what + " codes")
        assert_same_bytes(scale_bits(s), np.ascontiguousarray(so).view(np.uint32), what + " scales")
