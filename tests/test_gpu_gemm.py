"""GPU parity of the block-scaled FP8 GEMM against the oracle's exact
per-K-block value: |gpu - C*| <= 1e-3 * sum|a*b| (FP32 output), plus one
BF16 ulp of C* for BF16 output; no NaN or Inf.  The promotion of every
128-wide K interval with both block scales is the jp-study.kr page's
Figure 7(b); the Fprop, Dgrad and Wgrad shapes are Figure 6's linear-layer
GEMMs.

The oracle always quantizes the synthetic inputs itself; the GPU side uses
the GPU quantizers (whose bit-exactness is tested separately)."""
import numpy as np
import pytest
import torch

from fp8_fine_grained_quant_amd import synth
from helpers import check_gemm, per_tile_elements, sample_elements, to_dev, union_elements

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp8_fine_grained_quant_amd as fq
    return fq


def _rand_scaled(rng, shape, spread=3.0):
    return (rng.standard_normal(shape) * np.exp(rng.uniform(-spread, spread, (shape[0], 1)))).astype(
        np.float32)


def _full_check(fq, oracle, a, w, out_dtype, what):
    """Quantize a (1x128) and w (128x128) on both sides; compare all of C."""
    qa_o, sa_o = oracle.quant_1x128(a)
    qw_o, sw_o, _ = oracle.quant_128x128(w)
    c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qw_o, sw_o)
    qa, sa = fq.fp8_quant_1x128(to_dev(a))
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w))
    c = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return check_gemm(c.float().cpu().numpy(), c_ref, s_ref, out_dtype == torch.bfloat16, what)


def test_gemm_tiny_config_bf16(fq, oracle):
    a, w = synth.tiny_inputs()
    r = _full_check(fq, oracle, a, w, torch.bfloat16, "tiny fprop bf16")
    print(f"tiny: max |err| / tol = {r:.3g}")


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (1, 300, 256), (300, 200, 384), (256, 256, 128),
                                   (257, 513, 256), (512, 768, 1024), (33, 1000, 640),
                                   (1000, 40, 512), (127, 129, 128), (129, 127, 384)])
def test_gemm_shapes_and_tails(fq, oracle, M, N, K, out):
    rng = np.random.default_rng(M * 7 + N * 13 + K)
    a = _rand_scaled(rng, (M, K))
    w = _rand_scaled(rng, (N, K), 1.0) * np.float32(0.05)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    _full_check(fq, oracle, a, w, dt, f"{M}x{N}x{K} {out}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_row128_scales(fq, oracle, out):
    """ROW128: B carries one scale per row per 128 K (the weight-gradient
    layout, both operands quantized along the reduction dimension).  300 x 520
    runs on 256x224 tiles (the launcher's choice for this shape), whose
    epilogue stores 14 of the 16 chunks of a 256-byte row segment."""
    rng = np.random.default_rng(21)
    T, M, N = 640, 300, 520                 # reduction over T tokens
    dy = _rand_scaled(rng, (T, M))
    x = _rand_scaled(rng, (T, N))
    qa_o, sa_o = oracle.quant_1x128(dy, transposed=True)     # dY^T [M, T]
    qb_o, sb_o = oracle.quant_1x128(x, transposed=True)      # X^T  [N, T]
    c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qb_o, sb_o, mode=oracle.SCALE_ROW128)
    qa, sa = fq.fp8_quant_1x128(to_dev(dy), transposed=True)
    qb, sb = fq.fp8_quant_1x128(to_dev(x), transposed=True)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = fq.fp8_blockscaled_gemm(qa, sa, qb, sb, out_dtype=dt, scale_mode=fq.SCALE_ROW128)
    torch.cuda.synchronize()
    check_gemm(c.float().cpu().numpy(), c_ref, s_ref, out == "bf16", f"row128 {out}")


def test_gemm_transposed_weight_scales(fq, oracle):
    """Input-gradient shape: B = W^T codes from the 128x128 quantizer's
    transposed copy, its block scales read transposed through strides."""
    rng = np.random.default_rng(22)
    M, Nw, Kw = 384, 640, 384                # dX[M, Kw] = dY[M, Nw] * W[Nw, Kw]
    dy = _rand_scaled(rng, (M, Nw))
    w = _rand_scaled(rng, (Nw, Kw), 1.0) * np.float32(0.02)
    qa_o, sa_o = oracle.quant_1x128(dy)
    _, sw_o, qwt_o = oracle.quant_128x128(w, with_transpose=True)
    c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qwt_o, sw_o, sbs=(1, sw_o.shape[1]))
    qa, sa = fq.fp8_quant_1x128(to_dev(dy))
    _, sw, qwt = fq.fp8_quant_128x128(to_dev(w), with_transpose=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qwt, sw.t(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_gemm(c.cpu().numpy(), c_ref, s_ref, False, "dgrad-style")


def test_gemm_padding_untouched_and_repeatable(fq, oracle):
    rng = np.random.default_rng(23)
    M, N, K = 300, 260, 512
    a = _rand_scaled(rng, (M, K))
    w = _rand_scaled(rng, (N, K))
    qa, sa = fq.fp8_quant_1x128(to_dev(a))
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w))
    cbuf = torch.full((M, 272), float("nan"), dtype=torch.float32, device="cuda")
    c1 = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=torch.float32, c=cbuf[:, :N])
    torch.cuda.synchronize()
    assert torch.isnan(cbuf[:, N:]).all(), "ldc padding was written"
    c2 = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=torch.float32)
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32)), "not bitwise repeatable"
    qa_o, sa_o = oracle.quant_1x128(a)
    qw_o, sw_o, _ = oracle.quant_128x128(w)
    c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qw_o, sw_o)
    check_gemm(c2.cpu().numpy(), c_ref, s_ref, False, "padded")


def test_gemm_bf16_pitch_and_tail(fq, oracle):
    """BF16 output with a row pitch of 268 elements (536 bytes: every other
    row starts 8 but not 16 bytes aligned, so 16-byte chunks are stored as
    two 8-byte halves) and N = 261 (the last chunk of a row holds 5 columns).
    Values against the oracle; the pitch padding stays untouched."""
    rng = np.random.default_rng(29)
    M, N, K, ldc = 300, 261, 384, 268
    a = _rand_scaled(rng, (M, K))
    w = _rand_scaled(rng, (N, K), 1.0) * np.float32(0.05)
    qa, sa = fq.fp8_quant_1x128(to_dev(a))
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w))
    cbuf = torch.full((M, ldc), float("nan"), dtype=torch.bfloat16, device="cuda")
    c = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=torch.bfloat16, c=cbuf[:, :N])
    torch.cuda.synchronize()
    assert torch.isnan(cbuf[:, N:].float()).all(), "ldc padding was written"
    qa_o, sa_o = oracle.quant_1x128(a)
    qw_o, sw_o, _ = oracle.quant_128x128(w)
    c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qw_o, sw_o)
    check_gemm(c.float().cpu().numpy(), c_ref, s_ref, True, "bf16 pitch 268")


def test_gemm_zero_groups_and_extreme_scales(fq, oracle):
    """All-zero K blocks (scale +0) and activations spanning ~2^+-40 in one
    row: the promotion must not produce NaN/Inf and stays within tolerance."""
    rng = np.random.default_rng(24)
    M, N, K = 256, 256, 768
    a = rng.standard_normal((M, K)).astype(np.float32)
    a[:, 128:256] = 0.0
    a[:8] *= np.float32(2.0 ** 40)
    a[8:16] *= np.float32(2.0 ** -40)
    w = rng.standard_normal((N, K)).astype(np.float32)
    w[:128, 512:640] = 0.0
    _full_check(fq, oracle, a, w, torch.float32, "zero groups")


# --- the large configurations, on sampled outputs -------------------------------

def _sampled_check(fq, oracle, qa_o, sa_o, qb_o, sb_o, c, mode, sbs, bf16_out, seed, what):
    M, N = c.shape
    mi, ni = sample_elements(M, N, seed)
    c_ref, s_ref = oracle.gemm_exact_elems(qa_o, sa_o, qb_o, sb_o, mi, ni, mode=mode, sbs=sbs)
    cg = c.float()[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    assert torch.isfinite(c.float()).all(), f"{what}: non-finite output"
    r = check_gemm(cg, c_ref, s_ref, bf16_out, what)
    print(f"{what}: {mi.size} sampled elements, max |err| / tol = {r:.3g}")


def test_gemm_fprop_large(fq, oracle):
    a, w = synth.fprop_inputs()
    qa_o, sa_o = oracle.quant_1x128(a)
    qw_o, sw_o, _ = oracle.quant_128x128(w)
    qa, sa = fq.fp8_quant_1x128(to_dev(a))
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w))
    c = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _sampled_check(fq, oracle, qa_o, sa_o, qw_o, sw_o, c, oracle.SCALE_BLOCK128, None, True, 2,
                   "fprop 8192x18432x7168 bf16")


def test_gemm_dgrad_large(fq, oracle):
    dy, w = synth.dgrad_inputs()
    qa_o, sa_o = oracle.quant_1x128(dy)
    _, sw_o, qwt_o = oracle.quant_128x128(w, with_transpose=True)
    qa, sa = fq.fp8_quant_1x128(to_dev(dy))
    _, sw, qwt = fq.fp8_quant_128x128(to_dev(w), with_transpose=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qwt, sw.t(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    _sampled_check(fq, oracle, qa_o, sa_o, qwt_o, sw_o, c, oracle.SCALE_BLOCK128,
                   (1, sw_o.shape[1]), False, 3, "dgrad 8192x7168x18432 f32")


def test_gemm_wgrad_large(fq, oracle):
    dy, x = synth.wgrad_inputs()
    qa_o, sa_o = oracle.quant_1x128(dy, transposed=True)
    qb_o, sb_o = oracle.quant_1x128(x, transposed=True)
    qa, sa = fq.fp8_quant_1x128(to_dev(dy), transposed=True)
    qb, sb = fq.fp8_quant_1x128(to_dev(x), transposed=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qb, sb, out_dtype=torch.float32,
                                scale_mode=fq.SCALE_ROW128)
    torch.cuda.synchronize()
    _sampled_check(fq, oracle, qa_o, sa_o, qb_o, sb_o, c, oracle.SCALE_ROW128, None, False, 4,
                   "wgrad 2048x7168x8192 f32")


@pytest.mark.parametrize("N", [7168, 16384])
def test_gemm_row128_tile_widths(fq, oracle, N):
    """ROW128 GEMMs pick 256x224 or 256x256 tiles by the number of passes
    over 256 compute units: M = 2048 (8 tile rows) with N = 7168 gives 224
    tiles of 256 (one pass) or 256 tiles of 224 (one pass, narrower) -> 224;
    N = 16384 gives 512 tiles of 256 (two passes) or 592 of 224 (three) ->
    256.  Both widths against the oracle, on sampled outputs."""
    rng = np.random.default_rng(N)
    T, M = 256, 2048                        # reduction over T tokens
    dy = _rand_scaled(rng, (T, M))
    x = _rand_scaled(rng, (T, N))
    qa_o, sa_o = oracle.quant_1x128(dy, transposed=True)
    qb_o, sb_o = oracle.quant_1x128(x, transposed=True)
    qa, sa = fq.fp8_quant_1x128(to_dev(dy), transposed=True)
    qb, sb = fq.fp8_quant_1x128(to_dev(x), transposed=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qb, sb, out_dtype=torch.float32, scale_mode=fq.SCALE_ROW128)
    torch.cuda.synchronize()
    _sampled_check(fq, oracle, qa_o, sa_o, qb_o, sb_o, c, oracle.SCALE_ROW128, None, False, 5,
                   f"row128 2048x{N}x256")


@pytest.mark.parametrize("K,out", [(128, "bf16"), (256, "bf16"), (384, "bf16"), (384, "f32")])
def test_gemm_persistent_tile_loop(fq, oracle, K, out):
    """The GEMM runs one workgroup per compute unit, each looping over
    several 256x256 tiles; during a tile's last two K steps it already copies
    the next tile's first two.  8192 x 8192 is 1024 tiles (four per
    workgroup on 256 CUs).  K = 128: one step, so a plain prologue per tile;
    256: the copies switch to the next tile in the first step; 384: an odd
    step count, so the LDS stage of step 0 alternates from tile to tile.
    Oracle on sampled outputs, among them 4 random elements of every tile."""
    M = N = 8192
    rng = np.random.default_rng(K + 17)
    a = _rand_scaled(rng, (M, K))
    w = _rand_scaled(rng, (N, K), 1.0) * np.float32(0.05)
    qa_o, sa_o = oracle.quant_1x128(a)
    qw_o, sw_o, _ = oracle.quant_128x128(w)
    qa, sa = fq.fp8_quant_1x128(to_dev(a))
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w))
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=dt)
    torch.cuda.synchronize()
    mi, ni = union_elements(N, sample_elements(M, N, K), per_tile_elements([0], [M], N, K))
    c_ref, s_ref = oracle.gemm_exact_elems(qa_o, sa_o, qw_o, sw_o, mi, ni)
    assert torch.isfinite(c.float()).all(), "non-finite output"
    cg = c.float()[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    r = check_gemm(cg, c_ref, s_ref, out == "bf16", f"persistent 8192x8192x{K} {out}")
    print(f"8192x8192x{K} {out}: {mi.size} sampled elements, max |err| / tol = {r:.3g}")


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("T", [128, 384])
def test_gemm_persistent_row128(fq, oracle, T, pow2):
    """The ROW128 (weight-gradient) kernel through the persistent tile loop:
    2048 x 16384 is 512 tiles of 256x256 (two per workgroup), reduced over
    T = 128 tokens (one K step: a prologue per tile) or 384 (odd step count),
    with FP32 or power-of-two scales.  Oracle on sampled outputs, among them
    4 random elements of every tile."""
    M, N = 2048, 16384
    rng = np.random.default_rng(T + 31 + pow2)
    dy = _rand_scaled(rng, (T, M))
    x = _rand_scaled(rng, (T, N))
    rule = oracle.RULE_POW2 if pow2 else oracle.RULE_FP32
    qa_o, sa_o = oracle.quant_1x128(dy, transposed=True, rule=rule)
    qb_o, sb_o = oracle.quant_1x128(x, transposed=True, rule=rule)
    qa, sa = fq.fp8_quant_1x128(to_dev(dy), transposed=True, pow2=pow2)
    qb, sb = fq.fp8_quant_1x128(to_dev(x), transposed=True, pow2=pow2)
    c = fq.fp8_blockscaled_gemm(qa, sa, qb, sb, out_dtype=torch.float32, scale_mode=fq.SCALE_ROW128,
                                pow2=pow2)
    torch.cuda.synchronize()
    mi, ni = union_elements(N, sample_elements(M, N, T), per_tile_elements([0], [M], N, T))
    c_ref, s_ref = oracle.gemm_exact_elems(qa_o, sa_o, qb_o, sb_o, mi, ni, mode=oracle.SCALE_ROW128)
    assert torch.isfinite(c).all(), "non-finite output"
    cg = c[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    r = check_gemm(cg, c_ref, s_ref, False, f"row128 persistent T={T} pow2={pow2}")
    print(f"row128 2048x16384x{T} pow2={pow2}: {mi.size} sampled elements, max |err| / tol = {r:.3g}")


def test_gemm_persistent_pow2(fq, oracle):
    """Power-of-two scales through the persistent tile loop: 8192 x 8192 x 384
    (1024 tiles, odd step count), every tile sampled."""
    M = N = 8192
    K = 384
    rng = np.random.default_rng(77)
    a = _rand_scaled(rng, (M, K))
    w = _rand_scaled(rng, (N, K), 1.0) * np.float32(0.05)
    qa_o, sa_o = oracle.quant_1x128(a, rule=oracle.RULE_POW2)
    qw_o, sw_o, _ = oracle.quant_128x128(w, rule=oracle.RULE_POW2)
    qa, sa = fq.fp8_quant_1x128(to_dev(a), pow2=True)
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w), pow2=True)
    c = fq.fp8_blockscaled_gemm(qa, sa, qw, sw, out_dtype=torch.bfloat16, pow2=True)
    torch.cuda.synchronize()
    mi, ni = union_elements(N, sample_elements(M, N, 77), per_tile_elements([0], [M], N, 77))
    c_ref, s_ref = oracle.gemm_exact_elems(qa_o, sa_o, qw_o, sw_o, mi, ni)
    assert torch.isfinite(c.float()).all(), "non-finite output"
    cg = c.float()[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    r = check_gemm(cg, c_ref, s_ref, True, "pow2 persistent 8192x8192x384")
    print(f"pow2 8192x8192x384: {mi.size} sampled elements, max |err| / tol = {r:.3g}")


def test_gemm_random_shapes(fq, oracle):
    """40 seeded random cases: M, N in [1, 2600), K a multiple of 128 up to
    1024, row pitch N rounded up to 4 plus 0-8 elements, BF16 or FP32 out,
    BLOCK128 or ROW128 scales, FP32 or power-of-two scale rule, and rows
    scaled over up to e^+-4.  All of C against the oracle, padding
    untouched."""
    rng = np.random.default_rng(2024)
    for case in range(40):
        row, pow2, bf16 = rng.random() < 0.3, rng.random() < 0.3, rng.random() < 0.5
        K = 128 * int(rng.integers(1, 9))
        while True:
            M, N = int(rng.integers(1, 2600)), int(rng.integers(1, 2600))
            if M * N * K <= 3e8:
                break
        ldc = (N + 3) // 4 * 4 + 4 * int(rng.integers(0, 3))
        rule = oracle.RULE_POW2 if pow2 else oracle.RULE_FP32
        spread = rng.uniform(0, 4)
        if row:
            dy = (rng.standard_normal((K, M)) * np.exp(rng.uniform(-spread, spread, (K, 1)))).astype(np.float32)
            x = (rng.standard_normal((K, N)) * np.exp(rng.uniform(-spread, spread, (K, 1)))).astype(np.float32)
            qa_o, sa_o = oracle.quant_1x128(dy, transposed=True, rule=rule)
            qb_o, sb_o = oracle.quant_1x128(x, transposed=True, rule=rule)
            c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qb_o, sb_o, mode=oracle.SCALE_ROW128)
            qa, sa = fq.fp8_quant_1x128(to_dev(dy), transposed=True, pow2=pow2)
            qb, sb = fq.fp8_quant_1x128(to_dev(x), transposed=True, pow2=pow2)
            mode = fq.SCALE_ROW128
        else:
            a = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-spread, spread, (M, 1)))).astype(np.float32)
            w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
            qa_o, sa_o = oracle.quant_1x128(a, rule=rule)
            qb_o, sb_o, _ = oracle.quant_128x128(w, rule=rule)
            c_ref, s_ref = oracle.gemm_exact(qa_o, sa_o, qb_o, sb_o)
            qa, sa = fq.fp8_quant_1x128(to_dev(a), pow2=pow2)
            qb, sb, _ = fq.fp8_quant_128x128(to_dev(w), pow2=pow2)
            mode = fq.SCALE_BLOCK128
        dt = torch.bfloat16 if bf16 else torch.float32
        cbuf = torch.full((M, ldc), float("nan"), dtype=dt, device="cuda")
        c = fq.fp8_blockscaled_gemm(qa, sa, qb, sb, out_dtype=dt, c=cbuf[:, :N], scale_mode=mode,
                                    pow2=pow2)
        torch.cuda.synchronize()
        what = (f"case {case}: {'ROW128' if row else 'BLOCK128'} {M}x{N}x{K} ldc {ldc} "
                f"{'bf16' if bf16 else 'f32'} pow2={pow2}")
        assert torch.isnan(cbuf[:, N:].float()).all(), f"{what}: ldc padding was written"
        check_gemm(c.float().cpu().numpy(), c_ref, s_ref, bf16, what)
