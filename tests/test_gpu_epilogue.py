"""Bit-exact pin of the GEMM epilogue: FP32 output equals C* and BF16 output
equals C* rounded to nearest, ties to even ("Should Fixing Deepseek Take 60
Steps?", GEMM passage: FP8 operands in, BF16 or FP32 out; the rounding mode
is the reading stated with the tolerance).

The tolerance used by every other GEMM test (1e-3 * sum|a*b| plus one BF16
ulp) would also accept a truncating or round-half-up epilogue, so these
inputs are built to make C* an exact FP32 value that the kernel reaches
without rounding:
  * A row m holds E4M3 1.0 on one 16-wide segment (m % 8) of K blocks 0 and
    1, zero elsewhere; B column n holds, on segment s of block 0, the binary
    digits of an integer 256 <= H < 512 as E4M3 powers of two (sign shared),
    and on block 1 a single +-1 or 0 (delta).  So the block sums are
    P0 = +-H and P1 = delta, exact in any summation order (all products are
    powers of two within 8 binades of each other).
  * Scales are powers of two: sa[m, 0] = 2^e, sa[m, 1] = 2^(e-15), the B
    block scale 2^v per 128 columns, so
        C* = +-H * 2^(e+v) + delta * 2^(e+v-15),
    which needs 24 significant bits: exact in FP32, and every promotion step
    (an FMA with a power-of-two factor) is exact too.  Blocks 2.. carry zero
    codes (P = 0) under random power-of-two scales.
  * H odd with delta = 0 puts C* exactly halfway between two BF16 values
    (ulp 2 on [256, 512)); H = 1 (mod 4) must round down, H = 3 (mod 4) up
    (the even neighbour).  delta = +-1 moves C* one FP32 ulp off the tie.

Expected BF16 bits come from the definition (the nearer of the two
neighbouring BF16 values, ties to the even significand), cross-checked
against PyTorch's CPU FP32 -> BF16 cast.  The oracle's exact GEMM must agree
with the constructed C*, which checks the construction itself."""
import numpy as np
import pytest
import torch

SEG = 16            # K positions per selector segment
NSEG = 128 // SEG   # segments per K block


@pytest.fixture(scope="module")
def fq():  # noqa: D103
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp8_fine_grained_quant_amd as fq
    return fq


def _enc(oracle, v):
    v = np.asarray(v, dtype=np.float32)
    c = oracle.e4m3_encode(v).reshape(v.shape)
    assert np.array_equal(oracle.e4m3_decode(c).reshape(v.shape), v.astype(np.float64)), \
        "not exact in E4M3"
    return c


def _exact_case(oracle, M, N, K, seed, row_scales=False, e_range=(-30, 30), v_range=(-10, 10),
                with_delta=True):
    """Codes, scales and the exact C* (float64) of one constructed case.
    row_scales: B scales per column per K block (ROW128) instead of per
    128x128 block.  e_range / v_range: exponents of the block-0 A and B
    scales (half-open); with_delta=False leaves block 1 empty."""
    rng = np.random.default_rng(seed)
    nkb = K // 128
    assert nkb >= 2
    one = _enc(oracle, 1.0)
    qa = np.zeros((M, K), np.uint8)
    seg = np.arange(M) % NSEG
    for kb in (0, 1):
        for j in range(SEG):
            qa[np.arange(M), kb * 128 + seg * SEG + j] = one
    H = rng.integers(256, 512, (NSEG, N))
    sgn = rng.choice([-1.0, 1.0], (NSEG, N))
    delta = rng.choice([-1.0, 0.0, 0.0, 1.0], (NSEG, N)) if with_delta else np.zeros((NSEG, N))
    qb = np.zeros((N, K), np.uint8)
    for s in range(NSEG):
        qb[:, s * SEG] = _enc(oracle, sgn[s] * 256.0)
        for b in range(8):
            bit = ((H[s] - 256) >> b) & 1
            qb[:, s * SEG + 1 + (7 - b)] = np.where(bit == 1, _enc(oracle, sgn[s] * 2.0 ** b), 0)
        qb[:, 128 + s * SEG] = np.where(delta[s] != 0, _enc(oracle, delta[s]), 0)
    e = rng.integers(e_range[0], e_range[1], M)
    sa = np.empty((nkb, M), np.float32)
    sa[0] = np.ldexp(1.0, e)
    sa[1] = np.ldexp(1.0, e - 15)
    sa[2:] = np.ldexp(1.0, rng.integers(-20, 20, (nkb - 2, M)))
    nbn = (N + 127) // 128
    if row_scales:
        v_col = rng.integers(v_range[0], v_range[1], N)
        sb = np.empty((nkb, N), np.float32)
        sb[0] = sb[1] = np.ldexp(1.0, v_col)
        sb[2:] = np.ldexp(1.0, rng.integers(-20, 20, (nkb - 2, N)))
    else:
        v_blk = rng.integers(v_range[0], v_range[1], nbn)
        sb = np.empty((nbn, nkb), np.float32)
        sb[:, 0] = sb[:, 1] = np.ldexp(1.0, v_blk)
        sb[:, 2:] = np.ldexp(1.0, rng.integers(-20, 20, (nbn, nkb - 2)))
        v_col = v_blk[np.arange(N) // 128]
    ex = (e[:, None] + v_col[None, :]).astype(np.int64)
    s_of = seg[:, None]
    n_of = np.arange(N)[None, :]
    c_star = (np.ldexp(sgn[s_of, n_of] * H[s_of, n_of], ex)
              + np.ldexp(delta[s_of, n_of], ex - 15))
    assert np.array_equal(c_star.astype(np.float32).astype(np.float64), c_star), "C* not FP32"
    return qa, sa, qb, sb, c_star, H[s_of, n_of], delta[s_of, n_of]


def _bf16_rne_bits(c: np.ndarray) -> np.ndarray:
    """BF16 bit pattern nearest to each FP32-representable finite value
    (subnormals included: the neighbours are the bit patterns either side),
    ties to the even significand -- from the definition."""
    f = c.astype(np.float32)
    u = f.view(np.uint32)
    lo_bits = (u >> 16).astype(np.uint32)                      # toward zero
    hi_bits = lo_bits + 1                                       # away from zero
    lo = (lo_bits << 16).view(np.float32).astype(np.float64)
    hi = (hi_bits << 16).view(np.float32).astype(np.float64)
    d_lo = np.abs(c - lo)
    d_hi = np.abs(hi - c)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi_bits & 1) == 0))
    return np.where(pick_hi, hi_bits, lo_bits).astype(np.uint16)


def test_bf16_rne_definition_cases():
    """The definition above, on values fixed by hand, and against PyTorch
    (CPU only)."""
    vals = np.array([256.0, 257.0, 259.0, 257.0 + 2.0 ** -15, 257.0 - 2.0 ** -15, 259.0 - 2.0 ** -15,
                     -257.0, -259.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float64)
    want = np.array([256.0, 256.0, 260.0, 258.0, 256.0, 258.0, -256.0, -260.0, 1.0,
                     1.0 + 2.0 ** -6], np.float64)
    got = (_bf16_rne_bits(vals).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, want)
    t = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(t.view(np.uint16), _bf16_rne_bits(vals))
    # BF16 subnormals: ulp 2^-133; halfway cases go to the even pattern,
    # half the smallest one to zero
    u = 2.0 ** -133
    sub = np.array([3 * u, 2.5 * u, 3.5 * u, 0.5 * u, 0.75 * u, 1.5 * u, -2.5 * u], np.float64)
    want = np.array([3 * u, 2 * u, 4 * u, 0.0, u, 2 * u, -2 * u], np.float64)
    got = (_bf16_rne_bits(sub).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, want)
    t = torch.from_numpy(sub.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(t.view(np.uint16), _bf16_rne_bits(sub))


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K,row", [(256, 256, 384, False), (300, 264, 512, False),
                                       (256, 200, 256, True), (520, 300, 384, True)])
def test_epilogue_bits_exact(fq, oracle, M, N, K, row):
    qa, sa, qb, sb, c_star, H, delta = _exact_case(oracle, M, N, K, M + N + K + row, row)
    mode = oracle.SCALE_ROW128 if row else oracle.SCALE_BLOCK128
    c_o, _ = oracle.gemm_exact(qa, sa, qb, sb, mode=mode)
    assert np.array_equal(c_o, c_star), "oracle disagrees with the constructed C*"
    want_bf16 = _bf16_rne_bits(c_star)
    cpu = torch.from_numpy(c_star.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(cpu.view(np.uint16), want_bf16)
    tie = (H % 2 == 1) & (delta == 0)
    n_down = int((tie & (H % 4 == 1)).sum())
    n_up = int((tie & (H % 4 == 3)).sum())
    n_off = int(((H % 2 == 1) & (delta != 0)).sum())
    assert n_down > 50 and n_up > 50 and n_off > 50, (n_down, n_up, n_off)

    a = torch.from_numpy(qa).cuda()
    b = torch.from_numpy(qb).cuda()
    sa_d = torch.from_numpy(sa).cuda()
    sb_d = torch.from_numpy(sb).cuda()
    smode = fq.SCALE_ROW128 if row else fq.SCALE_BLOCK128
    c32 = fq.fp8_blockscaled_gemm(a, sa_d, b, sb_d, out_dtype=torch.float32, scale_mode=smode)
    c16 = fq.fp8_blockscaled_gemm(a, sa_d, b, sb_d, out_dtype=torch.bfloat16, scale_mode=smode)
    torch.cuda.synchronize()
    got32 = np.ascontiguousarray(c32.cpu().numpy()).view(np.uint32)
    want32 = c_star.astype(np.float32).view(np.uint32)
    bad = np.argwhere(got32 != want32)
    assert bad.size == 0, (f"FP32 output not exact at {len(bad)} elements, first {tuple(bad[0])}: "
                           f"{got32[tuple(bad[0])]:#x} want {want32[tuple(bad[0])]:#x}")
    got16 = np.ascontiguousarray(c16.view(torch.int16).cpu().numpy()).view(np.uint16)
    bad = np.argwhere(got16 != want_bf16)
    assert bad.size == 0, (f"BF16 output not RNE(C*) at {len(bad)} elements, first "
                           f"{tuple(bad[0])}: C* {c_star[tuple(bad[0])]!r} got "
                           f"{got16[tuple(bad[0])]:#06x} want {want_bf16[tuple(bad[0])]:#06x}")
    print(f"{M}x{N}x{K} row={row}: {n_down} ties down, {n_up} ties up, {n_off} one ulp off; "
          "FP32 and BF16 outputs bit-exact")


@pytest.mark.gpu
@pytest.mark.parametrize("row", [False, True])
def test_epilogue_bits_exact_subnormal(fq, oracle, row):
    """Outputs in the FP32 and BF16 subnormal range: block-0 scale exponents
    e + v in [-149, -130], so C* = +-H * 2^(e+v) runs from normal values down
    to a few FP32 ulps of 2^-149, every one exact in FP32 (the kernel's scale
    product and FMA are exact there unless denormals were flushed).  BF16
    rounds at its subnormal ulp 2^-133, with ties and underflow to zero."""
    M, N, K = 256, 256, 256
    qa, sa, qb, sb, c_star, _, _ = _exact_case(oracle, M, N, K, 4242 + row, row,
                                               e_range=(-74, -64), v_range=(-75, -65),
                                               with_delta=False)
    mode = oracle.SCALE_ROW128 if row else oracle.SCALE_BLOCK128
    c_o, _ = oracle.gemm_exact(qa, sa, qb, sb, mode=mode)
    assert np.array_equal(c_o, c_star), "oracle disagrees with the constructed C*"
    want_bf16 = _bf16_rne_bits(c_star)
    cpu = torch.from_numpy(c_star.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(cpu.view(np.uint16), want_bf16)
    mag = np.abs(c_star)
    sub32 = int(((mag > 0) & (mag < 2.0 ** -126)).sum())
    zero16 = int((want_bf16 & 0x7FFF == 0).sum())
    sub16 = int((((want_bf16 & 0x7F80) == 0) & ((want_bf16 & 0x7F) != 0)).sum())
    # exactly half a BF16 subnormal ulp (2^-133) from both neighbours
    ties = int(((mag < 2.0 ** -126) & (np.ldexp(mag, 134) % 2 == 1)).sum())
    assert sub32 > 1000 and zero16 > 50 and sub16 > 1000 and ties > 50, (sub32, zero16, sub16, ties)

    a = torch.from_numpy(qa).cuda()
    b = torch.from_numpy(qb).cuda()
    sa_d = torch.from_numpy(sa).cuda()
    sb_d = torch.from_numpy(sb).cuda()
    smode = fq.SCALE_ROW128 if row else fq.SCALE_BLOCK128
    c32 = fq.fp8_blockscaled_gemm(a, sa_d, b, sb_d, out_dtype=torch.float32, scale_mode=smode)
    c16 = fq.fp8_blockscaled_gemm(a, sa_d, b, sb_d, out_dtype=torch.bfloat16, scale_mode=smode)
    torch.cuda.synchronize()
    got32 = np.ascontiguousarray(c32.cpu().numpy()).view(np.uint32)
    want32 = c_star.astype(np.float32).view(np.uint32)
    bad = np.argwhere(got32 != want32)
    assert bad.size == 0, (f"FP32 output not exact at {len(bad)} elements, first {tuple(bad[0])}: "
                           f"{got32[tuple(bad[0])]:#x} want {want32[tuple(bad[0])]:#x}")
    got16 = np.ascontiguousarray(c16.view(torch.int16).cpu().numpy()).view(np.uint16)
    bad = np.argwhere(got16 != want_bf16)
    assert bad.size == 0, (f"BF16 output not RNE(C*) at {len(bad)} elements, first "
                           f"{tuple(bad[0])}: C* {c_star[tuple(bad[0])]!r} got "
                           f"{got16[tuple(bad[0])]:#06x} want {want_bf16[tuple(bad[0])]:#06x}")
    print(f"row={row}: {sub32} FP32 subnormal outputs, {sub16} BF16 subnormal, {zero16} BF16 zeros, "
          f"{ties} BF16 ties; bit-exact")


@pytest.mark.gpu
def test_epilogue_bits_exact_grouped(fq, oracle):
    """The grouped kernel's epilogue: three groups (one empty) over the same
    constructed rows, BF16 and FP32 out."""
    M, N, K = 600, 256, 256
    qa, sa, qb, sb, c_star, _, _ = _exact_case(oracle, M, N, K, 99)
    off = np.array([0, 250, 250, 600], np.int32)
    G = 3
    w = torch.from_numpy(np.stack([qb] * G)).cuda()
    sw = torch.from_numpy(np.stack([sb] * G)).cuda()
    offs = torch.from_numpy(off).cuda()
    a = torch.from_numpy(qa).cuda()
    sa_d = torch.from_numpy(sa).cuda()
    c32 = fq.fp8_grouped_gemm(a, sa_d, w, sw, offs, out_dtype=torch.float32)
    c16 = fq.fp8_grouped_gemm(a, sa_d, w, sw, offs, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(np.ascontiguousarray(c32.cpu().numpy()).view(np.uint32),
                          c_star.astype(np.float32).view(np.uint32)), "grouped FP32 not exact"
    assert np.array_equal(np.ascontiguousarray(c16.view(torch.int16).cpu().numpy()).view(np.uint16),
                          _bf16_rne_bits(c_star)), "grouped BF16 not RNE(C*)"
