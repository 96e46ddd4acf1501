"""The hot path under HIP graph capture.

Every entry point only enqueues kernels on the caller's stream: no host
synchronisation, no allocation and no memset (the bindings allocate only
when no output tensor is passed).  So a whole step -- the two quantizers and
the GEMM, or the MoE chain of quantize, dispatch and grouped GEMM -- can be
captured once into a graph and replayed.  Each replay is checked bit for bit
against the eager run; between replays the outputs are overwritten by eager
work and the stream is synchronised, so a replay that skipped a kernel or
replayed stale memory would be caught."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import fp8_fine_grained_quant_amd as fq
    return fq


def _poison(ts):
    for t in ts:
        if t.dtype == torch.uint8:
            t.fill_(0x55)
        else:
            t.fill_(float("nan"))


def _check_graph(step, outs, reps=3):
    step()                                  # eager reference (also fills host-side caches)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # a warm-up on a side stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(reps):
        _poison(outs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, t0) in enumerate(zip(outs, ref)):
            same = torch.equal(t.view(torch.uint8), t0.view(torch.uint8))
            assert same, f"replay {r}: output {i} differs from the eager run"


@pytest.mark.parametrize("pow2", [False, True])
def test_fprop_step_graph(fq, pow2):
    torch.manual_seed(1)
    M, N, K = 1024, 2304, 2048
    a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
    qa = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(K // 128, M, dtype=torch.float32, device="cuda")
    qw = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda")
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")

    def step():
        fq.fp8_quant_1x128(a, q=qa, s=sa, pow2=pow2)
        fq.fp8_quant_128x128(w, q=qw, s=sw, pow2=pow2)
        fq.fp8_blockscaled_gemm(qa, sa, qw, sw, c=c, pow2=pow2)

    _check_graph(step, [qa, sa, qw, sw, c])


def test_wgrad_step_graph(fq):
    torch.manual_seed(2)
    T, M, N = 1024, 512, 1536
    dy = torch.randn(T, M, device="cuda").to(torch.bfloat16)
    x = torch.randn(T, N, device="cuda").to(torch.bfloat16)
    qa = torch.empty(M, T, dtype=torch.uint8, device="cuda")
    sa = torch.empty(T // 128, M, dtype=torch.float32, device="cuda")
    qb = torch.empty(N, T, dtype=torch.uint8, device="cuda")
    sb = torch.empty(T // 128, N, dtype=torch.float32, device="cuda")
    c = torch.empty(M, N, dtype=torch.float32, device="cuda")

    def step():
        fq.fp8_quant_1x128(dy, transposed=True, q=qa, s=sa)
        fq.fp8_quant_1x128(x, transposed=True, q=qb, s=sb)
        fq.fp8_blockscaled_gemm(qa, sa, qb, sb, c=c, scale_mode=fq.SCALE_ROW128)

    _check_graph(step, [qa, sa, qb, sb, c])


def test_moe_step_graph(fq):
    rng = np.random.default_rng(3)
    T, K, N, G, topk = 512, 1024, 384, 8, 2
    counts = rng.multinomial(T * topk, np.full(G, 1.0 / G))
    counts[3] = 0                                            # an expert with no rows
    counts[0] += T * topk - counts.sum()
    rows = int(counts.sum())
    index = torch.from_numpy(rng.integers(0, T, rows).astype(np.int32)).cuda()
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    x = torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).cuda().to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((G * N, K)) * 0.02).astype(np.float32)).cuda().to(torch.bfloat16)
    q_tok = torch.empty(T, K, dtype=torch.uint8, device="cuda")
    s_tok = torch.empty(K // 128, T, dtype=torch.float32, device="cuda")
    q_g = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    s_g = torch.empty(K // 128, rows, dtype=torch.float32, device="cuda")
    qw = torch.empty(G * N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(G * N // 128, K // 128, dtype=torch.float32, device="cuda")
    c = torch.empty(rows, N, dtype=torch.bfloat16, device="cuda")

    def step():
        fq.fp8_quant_1x128(x, q=q_tok, s=s_tok)
        fq.fp8_dispatch_rows(q_tok, s_tok, index, q=q_g, s=s_g)
        fq.fp8_quant_128x128(w, q=qw, s=sw)            # the G experts' weights stacked: N % 128 == 0
        fq.fp8_grouped_gemm(q_g, s_g, qw.view(G, N, K), sw.view(G, N // 128, K // 128), offsets, c=c)

    _check_graph(step, [q_tok, s_tok, q_g, s_g, qw, sw, c])
