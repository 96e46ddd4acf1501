"""GPU parity of the power-of-two (E8M0) scale variant: quantizers bit-exact
against the oracle's power-of-two rule, GEMMs (whose matrix instruction
applies the scales and accumulates across K blocks) within the library
tolerance of the oracle's exact per-block value.  The pages ask for matrix
hardware that applies the group scales itself (why-be.why-be.co.kr page,
hardware-design passage)."""
import numpy as np
import pytest
import torch

from fp8_fine_grained_quant_amd import synth
from helpers import assert_same_bytes, check_gemm, codes, sample_elements, scale_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp8_fine_grained_quant_amd as fq
    return fq


def _spread(rng, shape, spread=4.0):
    return (rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, (shape[0], 1)))).astype(
        np.float32)


@pytest.mark.parametrize("shape", [(256, 512), (300, 200), (1, 128), (129, 1000)])
def test_pow2_quant_1x128(fq, oracle, shape):
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    x = _spread(rng, shape)
    x[0, :min(128, shape[1])] = 0.0                      # an all-zero group: s = 2^-127
    q_o, s_o = oracle.quant_1x128(x, rule=oracle.RULE_POW2)
    q, s = fq.fp8_quant_1x128(to_dev(x), pow2=True)
    assert_same_bytes(codes(q), q_o, "codes")
    assert_same_bytes(scale_bits(s), s_o.view(np.uint32), "scales")
    xt = np.ascontiguousarray(x.T)                      # 128x1 on the stored tensor
    qt_o, st_o = oracle.quant_1x128(xt, transposed=True, rule=oracle.RULE_POW2)
    qt, st = fq.fp8_quant_1x128(to_dev(xt), transposed=True, pow2=True)
    assert_same_bytes(codes(qt), qt_o, "128x1 codes")
    assert_same_bytes(scale_bits(st), st_o.view(np.uint32), "128x1 scales")


def test_pow2_quant_fprop_inputs(fq, oracle):
    a, w = synth.fprop_inputs()
    q_o, s_o = oracle.quant_1x128(a, rule=oracle.RULE_POW2)
    q, s = fq.fp8_quant_1x128(to_dev(a), pow2=True)
    assert_same_bytes(codes(q), q_o, "A codes")
    assert_same_bytes(scale_bits(s), s_o.view(np.uint32), "A scales")
    qw_o, sw_o, qt_o = oracle.quant_128x128(w, with_transpose=True, rule=oracle.RULE_POW2)
    qw, sw, qt = fq.fp8_quant_128x128(to_dev(w), with_transpose=True, pow2=True)
    assert_same_bytes(codes(qw), qw_o, "W codes")
    assert_same_bytes(scale_bits(sw), sw_o.view(np.uint32), "W scales")
    assert_same_bytes(codes(qt), qt_o, "W^T codes")


def _gemm_case(fq, oracle, a, w, out_dtype, what):
    qa_o, sa_o = oracle.quant_1x128(a, rule=oracle.RULE_POW2)
    qw_o, sw_o, _ = oracle.quant_128x128(w, rule=oracle.RULE_POW2)
    c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qw_o, sw_o)
    qa, sa = fq.fp8_quant_1x128(to_dev(a), pow2=True)
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w), pow2=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=out_dtype, pow2=True)
    torch.cuda.synchronize()
    return check_gemm(c.float().cpu().numpy(), c_ref, s_ref, out_dtype == torch.bfloat16, what)


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (300, 200, 384), (1, 300, 256), (513, 257, 1024)])
def test_pow2_gemm_shapes(fq, oracle, M, N, K, out):
    rng = np.random.default_rng(M + 7 * N + 13 * K)
    a = _spread(rng, (M, K))
    w = _spread(rng, (N, K), 1.0) * np.float32(0.05)
    _gemm_case(fq, oracle, a, w, torch.bfloat16 if out == "bf16" else torch.float32,
               f"pow2 {M}x{N}x{K} {out}")


def test_pow2_gemm_zero_groups_and_extreme_scales(fq, oracle):
    rng = np.random.default_rng(24)
    M, N, K = 256, 256, 768
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, 128:256] = 0.0
    a[:8] *= np.float32(2.0 ** 40)
    a[8:16] *= np.float32(2.0 ** -40)
    w = rng.standard_normal((N, K)).astype(np.float32)
    w[:128, 512:640] = 0.0
    _gemm_case(fq, oracle, a, w, torch.float32, "pow2 zero groups")


def test_pow2_gemm_row128_and_transposed_scales(fq, oracle):
    rng = np.random.default_rng(25)
    T, M, N = 640, 300, 520
    dy, x = _spread(rng, (T, M)), _spread(rng, (T, N))
    qa_o, sa_o = oracle.quant_1x128(dy, transposed=True, rule=oracle.RULE_POW2)
    qb_o, sb_o = oracle.quant_1x128(x, transposed=True, rule=oracle.RULE_POW2)
    c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qb_o, sb_o, mode=oracle.SCALE_ROW128)
    qa, sa = fq.fp8_quant_1x128(to_dev(dy), transposed=True, pow2=True)
    qb, sb = fq.fp8_quant_1x128(to_dev(x), transposed=True, pow2=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qb, sb, out_dtype=torch.float32,
                                scale_mode=fq.SCALE_ROW128, pow2=True)
    torch.cuda.synchronize()
    check_gemm(c.cpu().numpy(), c_ref, s_ref, False, "pow2 row128")
    # input-gradient shape: transposed weight codes, block scales read transposed
    M2, Nw, Kw = 384, 640, 384
    dy2 = _spread(rng, (M2, Nw))
    w = _spread(rng, (Nw, Kw), 1.0) * np.float32(0.02)
    qa_o, sa_o = oracle.quant_1x128(dy2, rule=oracle.RULE_POW2)
    _, sw_o, qwt_o = oracle.quant_128x128(w, with_transpose=True, rule=oracle.RULE_POW2)
    c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qwt_o, sw_o, sbs=(1, sw_o.shape[1]))
    qa, sa = fq.fp8_quant_1x128(to_dev(dy2), pow2=True)
    _, sw, qwt = fq.fp8_quant_128x128(to_dev(w), with_transpose=True, pow2=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qwt, sw.t(), out_dtype=torch.float32, pow2=True)
    torch.cuda.synchronize()
    check_gemm(c.cpu().numpy(), c_ref, s_ref, False, "pow2 dgrad-style")


def test_pow2_gemm_fprop_large(fq, oracle):
    a, w = synth.fprop_inputs()
    qa_o, sa_o = oracle.quant_1x128(a, rule=oracle.RULE_POW2)
    qw_o, sw_o, _ = oracle.quant_128x128(w, rule=oracle.RULE_POW2)
    qa, sa = fq.fp8_quant_1x128(to_dev(a), pow2=True)
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w), pow2=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=torch.bfloat16, pow2=True)
    torch.cuda.synchronize()
    M, N = c.shape
    mi, ni = sample_elements(M, N, 12)
    c_ref, s_ref = oracle.gemm_exact_elems(qa_o, sa_o, qw_o, sw_o, mi, ni)
    cg = c.float()[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    assert torch.isfinite(c.float()).all()
    r = check_gemm(cg, c_ref, s_ref, True, "pow2 fprop 8192x18432x7168")
    print(f"pow2 fprop: {mi.size} sampled, max |err| / tol = {r:.3g}")


def test_pow2_grouped(fq, oracle):
    rng = np.random.default_rng(26)
    counts = [0, 300, 1, 0, 257, 128]
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    Mt, G, N, K = int(off[-1]), len(counts), 384, 256
    x = _spread(rng, (Mt, K))
    w = (rng.standard_normal((G, N, K)) * 0.05).astype(np.float32)
    qa_o, sa_o = oracle.quant_1x128(x, rule=oracle.RULE_POW2)
    qw_o, sw_o, _ = oracle.quant_128x128(w.reshape(G * N, K), rule=oracle.RULE_POW2)
    qw_o, sw_o = qw_o.reshape(G, N, K), sw_o.reshape(G, N // 128, K // 128)
    mi, ni = np.meshgrid(np.arange(Mt), np.arange(N), indexing="ij")
    c_ref, s_ref = oracle.grouped_gemm_exact_elems(qa_o, sa_o, qw_o, sw_o, off, mi.ravel(),
                                                   ni.ravel())
    qa, sa = fq.fp8_quant_1x128(to_dev(x), pow2=True)
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w.reshape(G * N, K)), pow2=True)
    c = fq.fp8_grouped_gemm(qa, sa, qw.view(G, N, K), sw.view(G, N // 128, K // 128),
                            torch.from_numpy(off).cuda(), out_dtype=torch.float32, pow2=True)
    torch.cuda.synchronize()
    check_gemm(c.cpu().numpy().ravel(), c_ref, s_ref, False, "pow2 grouped")
