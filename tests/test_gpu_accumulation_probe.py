"""How many bits of the aligned products the gfx950 FP8 matrix instruction
keeps inside one 128-wide K block.

The pages give this as the reason for promotion: on H800 the FP8 tensor-core
accumulation keeps only about 14 bits of the aligned products
(why-be.why-be.co.kr page, accumulation-precision passage), so partial sums
are moved to FP32 at fixed K intervals (jp-study.kr page, Figure 7(b)).  On
gfx950 one instruction consumes a whole 128-wide K block, so the question
reduces to the instruction's own internal sum.

The probe goes through the public entry point fp8_blockscaled_gemm with
K = 128 and unit scales.  The promotion is then acc = 0 + P * 1, which is
exact, so each output element is the instruction's own FP32 result.  The
inputs are E4M3 codes with known exact dot products:
  * gap sweep: one large product 2^16 plus small products 2^(16-g), with the
    small terms after, before, or after a cancelling pair of large terms;
  * random codes over the whole E4M3 range, compared with the exact sum.
The expected values come from the oracle's exact per-block GEMM.  The only
contract asserted is the library's tolerance, |c - C*| <= 1e-3 * sum|a*b|;
the measured bit counts are printed for the design notes."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

K = 128
BIG_E = 8                      # a = b = 2^8: large product 2^16


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp8_fine_grained_quant_amd as fq
    return fq


def _code(oracle, v: float) -> int:
    c = int(oracle.e4m3_encode(np.array([v], dtype=np.float32))[0])
    assert float(oracle.e4m3_decode(np.array([c], dtype=np.uint8))[0]) == v, v
    return c


def _run(fq, qa: np.ndarray, qb: np.ndarray) -> np.ndarray:
    M, N = qa.shape[0], qb.shape[0]
    a = torch.from_numpy(qa).cuda()
    b = torch.from_numpy(qb).cuda()
    sa = torch.ones((1, M), dtype=torch.float32, device="cuda")
    sb = torch.ones((max(1, (N + 127) // 128), 1), dtype=torch.float32, device="cuda")
    c = fq.fp8_blockscaled_gemm(a, sa, b, sb, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return c.cpu().numpy().astype(np.float64)


PATTERNS = ("small_after", "small_after_x64", "small_before_x64", "cancel_then_small")


def _gap_inputs(oracle):
    """Rows (pattern, gap); column 0 reaches gaps 0..17 (b = 2^8 everywhere),
    column 1 gaps 17..34 (b = 2^-9 at the small positions)."""
    big = _code(oracle, 2.0 ** BIG_E)
    nbig = _code(oracle, -(2.0 ** BIG_E))
    qb = np.zeros((2, K), dtype=np.uint8)
    qb[0, :] = big
    qb[1, :] = _code(oracle, 2.0 ** -9)
    rows, meta = [], []
    for pat in PATTERNS:
        for g in range(0, 35):
            col = 0 if g <= 17 else 1
            e_small = (16 - g) - (BIG_E if col == 0 else -9)
            a = np.zeros(K, dtype=np.uint8)
            sm = _code(oracle, 2.0 ** e_small)
            # large terms only at k = 0, 1, 127; small terms at k = 3..66
            if pat == "small_after":
                big_pos, small_pos = [0], [3]
            elif pat == "small_after_x64":
                big_pos, small_pos = [0], list(range(3, 67))
            elif pat == "small_before_x64":
                big_pos, small_pos = [127], list(range(3, 67))
            else:
                big_pos, small_pos = [0], [3]
                a[1] = nbig
            for k in big_pos:
                a[k] = big
            for k in small_pos:
                a[k] = sm
            rows.append(a)
            meta.append((pat, g, col, len(small_pos)))
    qa = np.stack(rows)
    for k in (0, 1, 127):      # column 1: large products stay 2^16
        qb[1, k] = big
    return qa, qb, meta


def test_gap_sweep(fq, oracle):
    qa, qb, meta = _gap_inputs(oracle)
    c = _run(fq, qa, qb)
    sa = np.ones((1, qa.shape[0]), dtype=np.float32)
    sb = np.ones((1, 1), dtype=np.float32)
    c_ref, s_ref = oracle.gemm_exact(qa, sa, qb, sb)
    tol = 1e-3 * s_ref
    assert np.all(np.abs(c - c_ref) <= tol), "outside the library tolerance"
    lines = []
    for pat in PATTERNS:
        kept = []
        for i, (p, g, col, n) in enumerate(meta):
            if p != pat:
                continue
            exact, got = c_ref[i, col], c[i, col]
            small_total = n * 2.0 ** (16 - g)
            frac = (got - (exact - small_total)) / small_total
            kept.append((g, frac))
        first_loss = next((g for g, f in kept if abs(f - 1.0) > 1e-12), None)
        lines.append(f"{pat:18s} first gap with the small terms not fully kept: {first_loss}; "
                     + " ".join(f"{g}:{f:.3g}" for g, f in kept if 8 <= g <= 34))
    print("\n".join(["", "gfx950 FP8 MFMA 16x16x128, large product 2^16 + small products "
                     "2^(16-g); value = fraction of the small terms' sum kept"] + lines))


def test_position_sweep(fq, oracle):
    """Large product 2^16 at k = b0, one small product 2^-4 (gap 20) at k = p,
    for every p != b0: which K positions share the large term's truncation.
    Column c of B has 2^8 at its large position and 2^-9 elsewhere."""
    big = _code(oracle, 2.0 ** BIG_E)
    sm = _code(oracle, 2.0 ** 5)                 # 2^5 * 2^-9 = 2^-4
    starts = (0, 37)
    qb = np.full((len(starts), K), _code(oracle, 2.0 ** -9), dtype=np.uint8)
    for col, b0 in enumerate(starts):
        qb[col, b0] = big
    rows, meta = [], []
    for col, b0 in enumerate(starts):
        for p in range(K):
            if p == b0:
                continue
            a = np.zeros(K, dtype=np.uint8)
            a[b0], a[p] = big, sm
            rows.append(a)
            meta.append((col, b0, p))
    qa = np.stack(rows)
    c = _run(fq, qa, qb)
    c_ref, s_ref = oracle.gemm_exact(qa, np.ones((1, len(rows)), np.float32), qb,
                                     np.ones((1, 1), np.float32))
    assert np.all(np.abs(c - c_ref) <= 1e-3 * s_ref), "outside the library tolerance"
    for col, b0 in enumerate(starts):
        lost = [p for i, (cc, bb, p) in enumerate(meta) if cc == col and c[i, col] != c_ref[i, col]]
        print(f"\nlarge term at k={b0}: small term (gap 20) lost at k = {lost}")


def test_random_codes_effective_bits(fq, oracle):
    rng = np.random.default_rng(7)
    M = N = 256
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    qa = rng.choice(finite, size=(M, K)).astype(np.uint8)
    qb = rng.choice(finite, size=(N, K)).astype(np.uint8)
    c = _run(fq, qa, qb)
    sa = np.ones((1, M), dtype=np.float32)
    sb = np.ones((2, 1), dtype=np.float32)
    c_ref, s_ref = oracle.gemm_exact(qa, sa, qb, sb)
    assert np.all(np.abs(c - c_ref) <= 1e-3 * s_ref), "outside the library tolerance"
    da = oracle.e4m3_decode(qa).astype(np.float64)
    db = oracle.e4m3_decode(qb).astype(np.float64)
    maxprod = np.max(np.abs(da[:, None, :] * db[None, :, :]), axis=2)
    err = np.abs(c - c_ref)
    rel_max = err / maxprod
    rel_res = err / np.maximum(np.abs(c_ref), 1e-300)
    bits_max = -np.log2(np.maximum(rel_max, 2.0 ** -60))
    print(f"\nrandom E4M3 codes, {M * N} dot products of 128: exact {np.mean(err == 0) * 100:.1f} %; "
          f"error / largest product: max {rel_max.max():.3g} (>= {bits_max.min():.1f} bits), "
          f"median {np.median(rel_max):.3g}; error / |result|: median {np.median(rel_res):.3g}")
