"""GPU parity of the grouped (MoE expert) GEMM: the forward GEMM of the MoE
up-projection on activations quantized before dispatch (jp-study.kr page,
passage on FP8 dispatch and the up-projection), with per-expert 128x128 weight
scales.  Tolerance as for the dense GEMM."""
import numpy as np
import pytest
import torch

from fp8_fine_grained_quant_amd import synth
from helpers import (assert_same_bytes, check_gemm, codes, per_tile_elements, sample_elements,
                     scale_bits, to_dev, union_elements)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp8_fine_grained_quant_amd as fq
    return fq


def _offsets(counts):
    off = np.zeros(len(counts) + 1, dtype=np.int32)
    off[1:] = np.cumsum(counts)
    return off


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("counts,N,K", [([0, 300, 1, 0, 257, 128], 384, 256),
                                        ([5], 256, 128),
                                        ([0, 0, 513], 200, 384),
                                        ([1] * 40, 256, 256),
                                        ([127, 129, 0, 1], 129, 128)])
def test_grouped_small_full(fq, oracle, counts, N, K, out):
    rng = np.random.default_rng(len(counts) * 100 + N + K)
    off = _offsets(counts)
    Mt, G = int(off[-1]), len(counts)
    x = (rng.standard_normal((Mt, K)) * np.exp(rng.uniform(-3, 3, (Mt, 1)))).astype(np.float32)
    w = (rng.standard_normal((G, N, K)) * 0.05).astype(np.float32)
    qa_o, sa_o = oracle.quant_1x128(x)
    qw_o, sw_o, _ = oracle.quant_128x128(w.reshape(G * N, K))
    gn = (N + 127) // 128
    qw_o = qw_o.reshape(G, N, K)
    sw_o = sw_o.reshape(G, gn, K // 128) if N % 128 == 0 else None
    if sw_o is None:   # blocks straddle groups when N % 128 != 0: quantize per group
        qs = [oracle.quant_128x128(w[g]) for g in range(G)]
        qw_o = np.stack([q for q, _, _ in qs])
        sw_o = np.stack([s for _, s, _ in qs])
    mi, ni = np.meshgrid(np.arange(Mt), np.arange(N), indexing="ij")
    c_ref, s_ref = oracle.grouped_gemm_exact_elems(qa_o, sa_o, qw_o, sw_o, off, mi.ravel(),
                                                   ni.ravel())
    qa, sa = fq.fp8_quant_1x128(to_dev(x))
    wd = to_dev(w)
    qw = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    sw = torch.empty((G, gn, K // 128), dtype=torch.float32, device="cuda")
    for g in range(G):
        fq.fp8_quant_128x128(wd[g], q=qw[g], s=sw[g])
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    c = fq.fp8_grouped_gemm(qa, sa, qw, sw, torch.from_numpy(off).cuda(), out_dtype=dt)
    torch.cuda.synchronize()
    assert_same_bytes(codes(qw), qw_o, "expert weight codes")
    check_gemm(c.float().cpu().numpy().ravel(), c_ref, s_ref, out == "bf16", f"grouped {counts}")


def test_grouped_moe_config(fq, oracle):
    """256 experts, 32768 tokens x top-8 (Zipf 1.1 popularity, 4 experts
    forced empty), X_g[262144,7168] * W_e[2048,7168]^T, BF16 out.  Checked:
    the 1x128 codes/scales of every grouped row (via the gather identity
    quant(gather(X)) == gather(quant(X))), the 128x128 codes and scales of
    every expert weight in full, and C on 64 full rows, 64 full columns, 4096
    random elements, the first and last output tiles, and -- for every
    non-empty expert -- its first, last and 8 random rows in full (all 16
    column blocks)."""
    rt = synth.moe_routing_default()
    E, N, K = synth.MOE_EXPERTS, 2048, 7168
    off = rt.offsets
    Mt = int(off[-1])
    print(f"moe: {Mt} rows, {int((rt.counts == 0).sum())} empty experts, max {rt.counts.max()}",
          flush=True)
    xtok = synth.moe_tokens()
    w = synth.moe_expert_weights(range(E))                    # [E, N, K] bf16 bits
    # device side: gather, quantize, GEMM
    xg = to_dev(xtok)[torch.from_numpy(rt.token_of_row).cuda()]
    qa, sa = fq.fp8_quant_1x128(xg)
    del xg
    wd = to_dev(w.reshape(E * N, K))
    qw, sw, _ = fq.fp8_quant_128x128(wd)
    del wd
    c = fq.fp8_grouped_gemm(qa, sa, qw.view(E, N, K), sw.view(E, N // 128, K // 128),
                            torch.from_numpy(off).cuda(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    print("moe: gpu done", flush=True)
    # activations: oracle quantizes the 32768 token rows, rows are gathered
    qt_o, st_o = oracle.quant_1x128(xtok)
    assert_same_bytes(codes(qa), qt_o[rt.token_of_row], "grouped activation codes")
    assert_same_bytes(scale_bits(sa), st_o[:, rt.token_of_row].view(np.uint32),
                      "grouped activation scales")
    del qa, sa
    # weights: every expert in full, one expert at a time on the host
    qw_o = np.empty((E, N, K), dtype=np.uint8)
    sw_o = np.empty((E, N // 128, K // 128), dtype=np.float32)
    qw3 = qw.view(E, N, K)
    sw3 = sw.view(E, N // 128, K // 128)
    for e in range(E):
        q, s, _ = oracle.quant_128x128(w[e])
        qw_o[e], sw_o[e] = q, s
        assert_same_bytes(codes(qw3[e]), q, f"expert {e} weight codes")
        assert_same_bytes(scale_bits(sw3[e]), s.view(np.uint32), f"expert {e} weight scales")
    print("moe: expert weight codes and scales bit-exact", flush=True)
    del w
    # GEMM sample: the dense sample, plus first, last and 8 random full rows
    # of every non-empty expert
    rows = synth.expert_rows(off, 55)
    mi, ni = union_elements(N, sample_elements(Mt, N, 56),
                            (np.repeat(rows, N), np.tile(np.arange(N), rows.size)))
    c_ref, s_ref = oracle.grouped_gemm_exact_elems(qt_o[rt.token_of_row], st_o[:, rt.token_of_row],
                                                   qw_o, sw_o, off, mi, ni)
    cg = c.float()[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    r = check_gemm(cg, c_ref, s_ref, True, "moe grouped")
    print(f"moe: {mi.size} sampled elements ({rows.size} full expert rows), "
          f"max |err| / tol = {r:.3g}")


@pytest.mark.parametrize("K", [128, 384])
def test_grouped_persistent_tile_loop(fq, oracle, K):
    """Twelve groups of uneven size, three of them empty, 15,618 rows x 2048
    columns: 520 tiles, so workgroups (one per compute unit) run two or three
    tiles each, moving from group to group, with the next tile's first
    copies issued during the current one (K = 384, an odd step count) or a
    plain prologue per tile (K = 128).  Oracle on 4 random elements of every
    tile and on the first and last row of every group."""
    counts = [2048, 0, 1999, 2300, 0, 1, 2048, 777, 4096, 0, 300, 2049]
    N, G = 2048, len(counts)
    off = _offsets(counts)
    Mt = int(off[-1])
    rng = np.random.default_rng(K + 3)
    x = (rng.standard_normal((Mt, K)) * np.exp(rng.uniform(-3, 3, (Mt, 1)))).astype(np.float32)
    w = (rng.standard_normal((G * N, K)) * 0.05).astype(np.float32)
    qa_o, sa_o = oracle.quant_1x128(x)
    qw_o, sw_o, _ = oracle.quant_128x128(w)
    qa, sa = fq.fp8_quant_1x128(to_dev(x))
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w))
    c = fq.fp8_grouped_gemm(qa, sa, qw.view(G, N, K), sw.view(G, N // 128, K // 128),
                            torch.from_numpy(off).cuda(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    firsts = [(np.full(N, off[g]), np.arange(N)) for g in range(G) if counts[g]]
    lasts = [(np.full(N, off[g + 1] - 1), np.arange(N)) for g in range(G) if counts[g]]
    mi, ni = union_elements(N, per_tile_elements(off[:-1], off[1:], N, K), *firsts, *lasts)
    c_ref, s_ref = oracle.grouped_gemm_exact_elems(qa_o, sa_o, qw_o.reshape(G, N, K),
                                                   sw_o.reshape(G, N // 128, K // 128), off, mi, ni)
    assert torch.isfinite(c.float()).all(), "non-finite output"
    cg = c.float()[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    r = check_gemm(cg, c_ref, s_ref, True, f"grouped persistent K={K}")
    print(f"grouped {Mt} rows x {N} x {K}: {mi.size} sampled elements, max |err| / tol = {r:.3g}")


def test_grouped_many_empty_groups(fq, oracle):
    """4096 groups (the largest count the on-chip tile table holds), ten of
    them non-empty and scattered among long runs of empty ones: the tile ->
    group search steps over up to 64 empty table entries at a time.  263
    tiles, so the workgroups that run a second tile jump from the first
    groups to groups 3000, 4000 and 4095.  Oracle on 4 random elements of
    every tile and on the first and last row of every non-empty group."""
    G, N, K = 4096, 256, 128
    counts = np.zeros(G, dtype=np.int64)
    for g, n in [(0, 3), (63, 300), (64, 1), (65, 256), (1000, 513), (2047, 7), (2048, 129),
                 (3000, 64000), (4000, 260), (4095, 2)]:
        counts[g] = n
    off = _offsets(counts)
    Mt = int(off[-1])
    rng = np.random.default_rng(4096)
    x = (rng.standard_normal((Mt, K)) * np.exp(rng.uniform(-3, 3, (Mt, 1)))).astype(np.float32)
    nz = np.flatnonzero(counts)
    w = np.zeros((G, N, K), dtype=np.float32)
    w[nz] = (rng.standard_normal((nz.size, N, K)) * 0.05).astype(np.float32)
    qa_o, sa_o = oracle.quant_1x128(x)
    qw_o, sw_o, _ = oracle.quant_128x128(w.reshape(G * N, K))
    qa, sa = fq.fp8_quant_1x128(to_dev(x))
    qw, sw, _ = fq.fp8_quant_128x128(to_dev(w.reshape(G * N, K)))
    c = fq.fp8_grouped_gemm(qa, sa, qw.view(G, N, K), sw.view(G, N // 128, K // 128),
                            torch.from_numpy(off).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    firsts = [(np.full(N, off[g]), np.arange(N)) for g in nz]
    lasts = [(np.full(N, off[g + 1] - 1), np.arange(N)) for g in nz]
    mi, ni = union_elements(N, per_tile_elements(off[:-1], off[1:], N, 7), *firsts, *lasts)
    c_ref, s_ref = oracle.grouped_gemm_exact_elems(qa_o, sa_o, qw_o.reshape(G, N, K),
                                                   sw_o.reshape(G, N // 128, K // 128), off, mi, ni)
    assert torch.isfinite(c).all(), "non-finite output"
    cg = c[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().numpy()
    r = check_gemm(cg, c_ref, s_ref, False, "4096 groups")
    print(f"4096 groups, {Mt} rows, {mi.size} sampled elements: max |err| / tol = {r:.3g}")


def test_grouped_random(fq, oracle):
    """20 seeded random grouped GEMMs: 1-39 groups of 0-699 rows (a fifth of
    them forced empty), N a multiple of 128 up to 512, K up to 640, BF16 or
    FP32 out, FP32 or power-of-two scale rule.  All of C against the
    oracle."""
    rng = np.random.default_rng(777)
    for case in range(20):
        G = int(rng.integers(1, 40))
        N, K = int(rng.integers(1, 5)) * 128, 128 * int(rng.integers(1, 6))
        counts = rng.integers(0, 700, G) * (rng.random(G) < 0.8)
        off = _offsets(counts)
        Mt = int(off[-1])
        if Mt == 0:
            continue
        pow2, bf16 = rng.random() < 0.3, rng.random() < 0.5
        rule = oracle.RULE_POW2 if pow2 else oracle.RULE_FP32
        x = (rng.standard_normal((Mt, K)) * np.exp(rng.uniform(-3, 3, (Mt, 1)))).astype(np.float32)
        w = (rng.standard_normal((G * N, K)) * 0.05).astype(np.float32)
        qa_o, sa_o = oracle.quant_1x128(x, rule=rule)
        qw_o, sw_o, _ = oracle.quant_128x128(w, rule=rule)
        mi, ni = np.meshgrid(np.arange(Mt), np.arange(N), indexing="ij")
        c_ref, s_ref = oracle.grouped_gemm_exact_elems(qa_o, sa_o, qw_o.reshape(G, N, K),
                                                       sw_o.reshape(G, N // 128, K // 128), off,
                                                       mi.ravel(), ni.ravel())
        qa, sa = fq.fp8_quant_1x128(to_dev(x), pow2=pow2)
        qw, sw, _ = fq.fp8_quant_128x128(to_dev(w), pow2=pow2)
        dt = torch.bfloat16 if bf16 else torch.float32
        c = fq.fp8_grouped_gemm(qa, sa, qw.view(G, N, K), sw.view(G, N // 128, K // 128),
                                torch.from_numpy(off).cuda(), out_dtype=dt, pow2=pow2)
        torch.cuda.synchronize()
        check_gemm(c.float().cpu().numpy().ravel(), c_ref, s_ref, bf16,
                   f"case {case}: {G} groups, {Mt} rows, N {N}, K {K}, pow2={pow2}")
