"""Promotion-interval ablation on gfx950: promoting every 128-wide K block
into an FP32 register versus accumulating the whole K in the matrix
instruction's own accumulator.

The pages promote partial sums to FP32 at a fixed K interval because the
H800 tensor-core accumulation keeps only about 14 bits of the aligned
products (why-be.why-be.co.kr page, accumulation-precision passage;
jp-study.kr page, Figure 7(b)).  Both variants are public entry points:
  * fp8_blockscaled_gemm: each K block's instruction result is a fresh
    partial sum, promoted with an FP32 FMA (interval 128);
  * fp8_blockscaled_gemm_pow2 with unit scales (E8M0 exponent 0): every K
    block accumulates onto the previous result inside the instruction
    (no promotion; the interval is the whole K).
With all scales 1 both compute the same exact value C* = A * B^T, which the
oracle gives in fp64.  Inputs: E4M3 codes of N(0, 40) values (the whole
code range, saturated at 448), M = N = 256, K = 128, 1024, 7168.  Both are
held to the library tolerance; the medians of |err| / |C*| are printed for
the design notes."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp8_fine_grained_quant_amd as fq
    return fq


@pytest.mark.parametrize("K", [128, 1024, 7168])
def test_promotion_interval(fq, oracle, K):
    M = N = 256
    rng = np.random.default_rng(K + 5)
    qa = oracle.e4m3_encode(np.clip(rng.standard_normal((M, K)) * 40, -448, 448).astype(np.float32))
    qb = oracle.e4m3_encode(np.clip(rng.standard_normal((N, K)) * 40, -448, 448).astype(np.float32))
    qa = qa.reshape(M, K)
    qb = qb.reshape(N, K)
    sa = np.ones((K // 128, M), np.float32)
    sb = np.ones((N // 128, K // 128), np.float32)
    c_ref, s_ref = oracle.gemm_exact(qa, sa, qb, sb)
    a, b = torch.from_numpy(qa).cuda(), torch.from_numpy(qb).cuda()
    sa_d, sb_d = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda()
    c_prom = fq.fp8_blockscaled_gemm(a, sa_d, b, sb_d, out_dtype=torch.float32)
    c_acc = fq.fp8_blockscaled_gemm(a, sa_d, b, sb_d, out_dtype=torch.float32, pow2=True)
    torch.cuda.synchronize()
    res = {}
    for name, c in (("promote every 128", c_prom), ("accumulate in the instruction", c_acc)):
        g = c.cpu().numpy().astype(np.float64)
        from helpers import check_gemm
        r = check_gemm(g, c_ref, s_ref, False, f"{name}, K={K}")
        nz = c_ref != 0
        rel = np.abs(g - c_ref)[nz] / np.abs(c_ref[nz])
        res[name] = (float(np.median(rel)), float(rel.max()), r)
    for name, (med, mx, r) in res.items():
        print(f"K={K:5d} {name:30s}: median |err|/|C*| {med:.3g}, max {mx:.3g}, "
              f"max |err|/tol {r:.3g}")
