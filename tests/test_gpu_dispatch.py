"""GPU parity of the FP8 dispatch permutation (jp-study.kr page, passage on
quantizing the MoE up-projection's activations before dispatch and
dispatching them in FP8).  Expected rows come from the oracle: the codes and
scales of the gathered tokens, which the 1x128 quantizer's row locality makes
equal to the gather of the quantized tokens (quantize-then-gather ==
gather-then-quantize, pinned for the oracle on the CPU).  Everything is
compared bit for bit."""
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


def _tokens(rng, T, C):
    return (rng.standard_normal((T, C)) * np.exp(rng.uniform(-4, 4, (T, 1)))).astype(np.float32)


@pytest.mark.parametrize("T,C,R", [(100, 640, 300), (37, 200, 90), (5, 7168, 64), (1, 128, 3)])
def test_dispatch_small_full(fq, oracle, T, C, R):
    rng = np.random.default_rng(T * 1000 + C + R)
    x = _tokens(rng, T, C)
    index = rng.integers(0, T, R).astype(np.int32)
    qg_o, sg_o = oracle.quant_1x128(x[index])           # quantize the gathered rows
    qt, st = fq.fp8_quant_1x128(to_dev(x))
    qg, sg = fq.fp8_dispatch_rows(qt, st, torch.from_numpy(index).cuda())
    torch.cuda.synchronize()
    assert_same_bytes(codes(qg), qg_o, "dispatched codes")
    assert_same_bytes(scale_bits(sg), np.ascontiguousarray(sg_o).view(np.uint32), "dispatched scales")


def test_dispatch_skips_out_of_range_and_keeps_padding(fq, oracle):
    rng = np.random.default_rng(9)
    T, C, R = 50, 384, 40
    x = _tokens(rng, T, C)
    index = rng.integers(0, T, R).astype(np.int32)
    index[[3, 17, 39]] = [-1, T, 2 ** 31 - 1]
    qt, st = fq.fp8_quant_1x128(to_dev(x))
    qbuf = torch.full((R, C + 32), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((3, R + 8), float("nan"), dtype=torch.float32, device="cuda")
    fq.fp8_dispatch_rows(qt, st, torch.from_numpy(index).cuda(), q=qbuf[:, :C], s=sbuf[:, :R])
    torch.cuda.synchronize()
    q, s = codes(qbuf), sbuf.cpu().numpy()
    assert (q[:, C:] == 0xAB).all(), "code padding written"
    assert np.isnan(s[:, R:]).all(), "scale padding written"
    bad = np.isin(np.arange(R), [3, 17, 39])
    assert (q[bad, :C] == 0xAB).all() and np.isnan(s[:, :R][:, bad]).all(), "skipped rows written"
    good = ~bad
    qg_o, sg_o = oracle.quant_1x128(x[index[good]])
    assert_same_bytes(q[good, :C], qg_o, "dispatched codes")
    assert_same_bytes(np.ascontiguousarray(s[:, :R][:, good]).view(np.uint32),
                      np.ascontiguousarray(sg_o).view(np.uint32), "dispatched scales")


def test_dispatch_empty(fq):
    qt = torch.zeros((4, 256), dtype=torch.uint8, device="cuda")
    st = torch.zeros((2, 4), dtype=torch.float32, device="cuda")
    q, s = fq.fp8_dispatch_rows(qt, st, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert q.shape == (0, 256) and s.shape == (2, 0)


def test_dispatch_moe_config(fq, oracle):
    """32768 tokens x 7168 channels dispatched into 262144 expert-ordered
    rows (top-8 routing); checked on a seeded sample of rows plus the first
    and last row of every non-empty expert."""
    r = synth.moe_routing_default()
    xt = synth.moe_tokens()
    index = r.token_of_row.astype(np.int32)
    R = index.size
    rng = np.random.default_rng(77)
    rows = np.concatenate([rng.choice(R, 4096, replace=False),
                           r.offsets[:-1][r.counts > 0], r.offsets[1:][r.counts > 0] - 1])
    rows = np.unique(rows)
    qt, st = fq.fp8_quant_1x128(to_dev(xt))
    qg, sg = fq.fp8_dispatch_rows(qt, st, torch.from_numpy(index).cuda())
    torch.cuda.synchronize()
    sel = torch.from_numpy(rows).cuda()
    qs = codes(qg[sel])
    ss = np.ascontiguousarray(sg[:, sel].cpu().numpy())
    qg_o, sg_o = oracle.quant_1x128(xt[index[rows]])
    assert_same_bytes(qs, qg_o, "dispatched codes (sample)")
    assert_same_bytes(ss.view(np.uint32), np.ascontiguousarray(sg_o).view(np.uint32),
                      "dispatched scales (sample)")


def test_dispatch_random(fq, oracle):
    """30 seeded random dispatches, bit for bit: T tokens up to 600, widths
    up to 3000 (ragged, and aligned or not to 16 bytes), up to 1500 output
    rows drawn from the tokens with repeats, 2 % of them out of range (left
    unwritten)."""
    rng = np.random.default_rng(3131)
    for case in range(30):
        T, C, R = int(rng.integers(1, 600)), int(rng.integers(1, 3000)), int(rng.integers(1, 1500))
        x = _tokens(rng, T, C)
        index = rng.integers(0, T, R).astype(np.int32)
        bad = rng.random(R) < 0.02
        index[bad] = rng.choice(np.array([-1, T, 2 ** 31 - 1], dtype=np.int32), int(bad.sum()))
        qt, st = fq.fp8_quant_1x128(to_dev(x))
        G = (C + 127) // 128
        qbuf = torch.full((R, C), 0xAB, dtype=torch.uint8, device="cuda")
        sbuf = torch.full((G, R), float("nan"), dtype=torch.float32, device="cuda")
        fq.fp8_dispatch_rows(qt, st, torch.from_numpy(index).cuda(), q=qbuf, s=sbuf)
        torch.cuda.synchronize()
        q, s = codes(qbuf), sbuf.cpu().numpy()
        what = f"case {case}: T {T} C {C} R {R}"
        assert (q[bad] == 0xAB).all() and np.isnan(s[:, bad]).all(), what + ": skipped rows written"
        good = ~bad
        if good.any():
            qg_o, sg_o = oracle.quant_1x128(x[index[good]])
            assert_same_bytes(q[good], qg_o, what + " codes")
            assert_same_bytes(s[:, good].view(np.uint32), np.ascontiguousarray(sg_o).view(np.uint32),
                              what + " scales")
