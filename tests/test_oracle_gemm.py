"""Pins for the oracle's block-scaled GEMM.

Method (jp-study.kr page, Figure 7(b); "Should Fixing Deepseek Take 60
Steps?", GEMM passage): the FP8 GEMM takes E4M3 operands; each 128-wide K
interval's partial result is multiplied by the activation tile scale and the
weight block scale and accumulated in FP32 ("promotion"); output BF16 or
FP32.  The oracle computes the exact value of
that sum (fp64, each per-block partial exact); these tests check it against
exact rational arithmetic, integer matmul and structural identities.
"""
from fractions import Fraction

import numpy as np
import pytest


def _dec_exact(c: int) -> Fraction:
    if (c & 0x7F) == 0x7F:
        raise ValueError("NaN code")
    e, m = (c >> 3) & 15, c & 7
    mag = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -mag if c & 0x80 else mag


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x30
    return c


def _rand_scales(rng, shape):
    return (rng.uniform(0.5, 2.0, size=shape) * np.exp2(rng.integers(-20, 4, size=shape))).astype(
        np.float32)


def _fraction_gemm(qa, sa, qb, sb_of):
    """Exact C and S with Python rationals.  sb_of(n, kb) -> FP32 scale."""
    M, K = qa.shape
    N = qb.shape[0]
    da = [[_dec_exact(int(v)) for v in row] for row in qa]
    db = [[_dec_exact(int(v)) for v in row] for row in qb]
    C = np.empty((M, N), dtype=object)
    S = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            c = Fraction(0)
            s = Fraction(0)
            for kb in range(K // 128):
                sab = Fraction(float(sa[kb, m])) * Fraction(float(sb_of(n, kb)))
                part = sum((da[m][k] * db[n][k] for k in range(kb * 128, kb * 128 + 128)),
                           Fraction(0))
                pabs = sum((abs(da[m][k] * db[n][k]) for k in range(kb * 128, kb * 128 + 128)),
                           Fraction(0))
                c += sab * part
                s += abs(sab) * pabs
            C[m, n] = c
            S[m, n] = s
    return C, S


def _check_close_to_exact(c, s, C, S):
    for idx in np.ndindex(C.shape):
        # the oracle rounds once per K block (scale product times partial) and
        # once per accumulation: a few fp64 ulps of S
        err = abs(Fraction(float(c[idx])) - C[idx])
        assert err <= Fraction(2) ** -48 * S[idx] + Fraction(2) ** -1000, (idx, float(err))
        assert abs(Fraction(float(s[idx])) - S[idx]) <= Fraction(2) ** -48 * S[idx]


@pytest.mark.parametrize("K", [128, 256, 384])
def test_gemm_block128_vs_exact_rationals(oracle, K):
    rng = np.random.default_rng(K)
    M, N = 5, 3
    qa = _rand_codes(rng, (M, K))
    qb = _rand_codes(rng, (N, K))
    sa = _rand_scales(rng, (K // 128, M))
    sb = _rand_scales(rng, (1, K // 128))
    c, s = oracle.gemm_exact(qa, sa, qb, sb)
    C, S = _fraction_gemm(qa, sa, qb, lambda n, kb: sb[n // 128, kb])
    _check_close_to_exact(c, s, C, S)


def test_gemm_block128_second_n_block_and_strides(oracle):
    """N spans two 128-blocks; the B scales are read through strides
    (transposed storage), as for a weight used in the backward pass."""
    rng = np.random.default_rng(1)
    K, M = 256, 2
    n_idx = [0, 127, 128, 129, 200]
    qa = _rand_codes(rng, (M, K))
    qb = _rand_codes(rng, (256, K))
    sa = _rand_scales(rng, (K // 128, M))
    sbT = _rand_scales(rng, (K // 128, 2))          # stored [kb][n/128]
    c, s = oracle.gemm_exact(qa, sa, qb, sbT, sbs=(1, 2))
    C, S = _fraction_gemm(qa, sa, qb[n_idx], lambda j, kb: sbT[kb, n_idx[j] // 128])
    _check_close_to_exact(c[:, n_idx], s[:, n_idx], C, S)


def test_gemm_row128_vs_exact_rationals(oracle):
    rng = np.random.default_rng(2)
    M, N, K = 4, 6, 256
    qa = _rand_codes(rng, (M, K))
    qb = _rand_codes(rng, (N, K))
    sa = _rand_scales(rng, (K // 128, M))
    sb = _rand_scales(rng, (K // 128, N))
    c, s = oracle.gemm_exact(qa, sa, qb, sb, mode=oracle.SCALE_ROW128)
    C, S = _fraction_gemm(qa, sa, qb, lambda n, kb: sb[kb, n])
    _check_close_to_exact(c, s, C, S)


def test_gemm_integer_codes_equal_int_matmul(oracle):
    """Codes whose values are small integers and unit scales: the result is an
    integer matmul, computed exactly by numpy in int64."""
    rng = np.random.default_rng(3)
    int_codes = {0x38: 1, 0x40: 2, 0x44: 3, 0x48: 4, 0x4A: 5, 0x4C: 6, 0x4E: 7, 0x50: 8,
                 0x00: 0, 0xB8: -1, 0xC0: -2, 0xC4: -3, 0xC8: -4}
    keys = np.array(list(int_codes.keys()), dtype=np.uint8)
    vals = np.array(list(int_codes.values()), dtype=np.int64)
    M, N, K = 64, 48, 512
    ia = rng.integers(0, len(keys), size=(M, K))
    ib = rng.integers(0, len(keys), size=(N, K))
    c, s = oracle.gemm_exact(keys[ia], np.ones((K // 128, M), np.float32), keys[ib],
                             np.ones((1, K // 128), np.float32))
    ref = vals[ia] @ vals[ib].T
    assert np.array_equal(c, ref.astype(np.float64))
    assert np.array_equal(s, (np.abs(vals[ia]) @ np.abs(vals[ib]).T).astype(np.float64))


def test_gemm_identity_b_returns_dequantized_a(oracle):
    rng = np.random.default_rng(4)
    M, K = 16, 256
    qa = _rand_codes(rng, (M, K))
    sa = _rand_scales(rng, (K // 128, M))
    qb = np.zeros((K, K), dtype=np.uint8)
    qb[np.arange(K), np.arange(K)] = 0x38                      # 1.0 on the diagonal
    c, _ = oracle.gemm_exact(qa, sa, qb, np.ones((2, 2), np.float32))
    deq = oracle.e4m3_decode(qa) * np.repeat(sa.T.astype(np.float64), 128, axis=1)
    assert np.array_equal(c, deq)


def test_gemm_single_k_block_isolates_scale_indexing(oracle):
    rng = np.random.default_rng(5)
    M, N, K = 8, 256, 512
    for kb0 in range(K // 128):
        qa = np.zeros((M, K), np.uint8)
        qb = np.zeros((N, K), np.uint8)
        qa[:, kb0 * 128:(kb0 + 1) * 128] = _rand_codes(rng, (M, 128))
        qb[:, kb0 * 128:(kb0 + 1) * 128] = _rand_codes(rng, (N, 128))
        sa = _rand_scales(rng, (K // 128, M))
        sb = _rand_scales(rng, (2, K // 128))
        c, _ = oracle.gemm_exact(qa, sa, qb, sb)
        part = oracle.e4m3_decode(qa) @ oracle.e4m3_decode(qb).T      # exact: one block
        sab = sa[kb0][:, None].astype(np.float64) * np.repeat(sb[:, kb0], 128)[None, :]
        assert np.array_equal(c, sab * part)


def test_gemm_row128_equals_block128_for_blockwise_constant_scales(oracle):
    rng = np.random.default_rng(6)
    M, N, K = 16, 256, 384
    qa = _rand_codes(rng, (M, K))
    qb = _rand_codes(rng, (N, K))
    sa = _rand_scales(rng, (K // 128, M))
    sblk = _rand_scales(rng, (2, K // 128))
    srow = np.repeat(sblk.T, 128, axis=1)                         # [kb][n]
    c1, s1 = oracle.gemm_exact(qa, sa, qb, sblk)
    c2, s2 = oracle.gemm_exact(qa, sa, qb, srow, mode=oracle.SCALE_ROW128)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_gemm_elems_equal_full(oracle):
    rng = np.random.default_rng(7)
    M, N, K = 40, 300, 256
    qa = _rand_codes(rng, (M, K))
    qb = _rand_codes(rng, (N, K))
    sa = _rand_scales(rng, (K // 128, M))
    sb = _rand_scales(rng, (3, K // 128))
    c, s = oracle.gemm_exact(qa, sa, qb, sb)
    mi = rng.integers(0, M, 500)
    ni = rng.integers(0, N, 500)
    ce, se = oracle.gemm_exact_elems(qa, sa, qb, sb, mi, ni)
    assert np.array_equal(ce, c[mi, ni]) and np.array_equal(se, s[mi, ni])


def test_grouped_gemm_equals_per_group_dense(oracle):
    rng = np.random.default_rng(8)
    G, N, K = 5, 256, 256
    counts = np.array([3, 0, 130, 1, 0])
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    Mt = int(offsets[-1])
    qa = _rand_codes(rng, (Mt, K))
    sa = _rand_scales(rng, (K // 128, Mt))
    qw = _rand_codes(rng, (G, N, K))
    sw = _rand_scales(rng, (G, 2, K // 128))
    mi, ni = np.meshgrid(np.arange(Mt), np.arange(N), indexing="ij")
    c, s = oracle.grouped_gemm_exact_elems(qa, sa, qw, sw, offsets, mi.ravel(), ni.ravel())
    c = c.reshape(Mt, N)
    for g in range(G):
        r0, r1 = offsets[g], offsets[g + 1]
        if r0 == r1:
            continue
        ref, _ = oracle.gemm_exact(qa[r0:r1], np.ascontiguousarray(sa[:, r0:r1]), qw[g], sw[g])
        assert np.array_equal(c[r0:r1], ref), g


def test_grouped_gemm_vs_exact_rationals(oracle):
    rng = np.random.default_rng(9)
    G, N, K = 3, 4, 128
    offsets = np.array([0, 2, 2, 4], np.int32)
    qa = _rand_codes(rng, (4, K))
    sa = _rand_scales(rng, (1, 4))
    qw = _rand_codes(rng, (G, N, K))
    sw = _rand_scales(rng, (G, 1, 1))
    mi, ni = np.meshgrid(np.arange(4), np.arange(N), indexing="ij")
    c, s = oracle.grouped_gemm_exact_elems(qa, sa, qw, sw, offsets, mi.ravel(), ni.ravel())
    for m in range(4):
        g = 0 if m < 2 else 2
        C, S = _fraction_gemm(qa[m:m + 1], sa[:, m:m + 1], qw[g], lambda n, kb: sw[g, 0, kb])
        _check_close_to_exact(c.reshape(4, N)[m:m + 1], s.reshape(4, N)[m:m + 1], C, S)


def test_bf16_ulp_and_tolerance(oracle):
    u = oracle.bf16_ulp(np.array([1.0, 1.5, 1.99, 2.0, 448.0, -3.0, 2.0 ** -130, 0.0]))
    assert u.tolist() == [2.0 ** -7, 2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0, 2.0 ** -6,
                          2.0 ** -133, 2.0 ** -133]
    tol = oracle.gemm_tolerance(np.array([1.0]), np.array([10.0]), bf16_out=True)
    assert tol[0] == 1e-2 + 2.0 ** -7
