"""Seeded synthetic inputs for the fine-grained FP8 quantize + GEMM path.

This module only draws numbers; it holds none of the method's arithmetic
(no scaling, no encoding, no products).  Both the HIP path (through the tests
and the benchmark) and the CPU oracle consume the arrays it returns, so the
two sides always see identical inputs.

Recipe (shared by every workload):
  * values are drawn as float32 from ``numpy.random.default_rng(seed)``:
    ``standard_normal * std``;
  * outliers: ``round(frac * numel)`` positions chosen uniformly without
    replacement from the same generator, multiplied by ``factor`` -- the
    activation outliers that make per-tensor scaling fragile ("Should
    Fixing Deepseek Take 60 Steps?", max-abs scaling passage);
  * BF16 tensors are the float32 draw rounded to nearest-even BF16; they are
    returned as uint16 bit patterns (numpy has no bfloat16).
MoE routing: expert popularity p_e proportional to rank_e^-1.1 (Zipf), ranks a
seeded permutation; a few seeded experts are banned (p = 0) so that empty
experts occur; every token draws ``top_k`` distinct experts in proportion to
p (Gumbel-top-k); rows are ordered by (expert, token).
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os

import numpy as np


def normal_f32(shape, std: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_with_outliers(shape, std: float, seed: int, frac: float = 0.0,
                         factor: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if frac > 0.0:
        n = x.size
        count = int(round(frac * n))
        idx = rng.choice(n, size=count, replace=False)
        flat = x.reshape(-1)
        flat[idx] *= np.float32(factor)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to nearest-even BF16; return the uint16 bit patterns.

    NaN is not expected in synthetic inputs and is not handled specially."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


# --- MoE routing --------------------------------------------------------------

@dataclasses.dataclass
class Routing:
    offsets: np.ndarray      # int32[E+1], rows of expert e are [offsets[e], offsets[e+1])
    token_of_row: np.ndarray  # int64[T*top_k], source token of each grouped row
    counts: np.ndarray       # int64[E]
    banned: np.ndarray       # experts forced empty


def moe_routing(num_experts: int, num_tokens: int, top_k: int, zipf_s: float, seed: int,
                num_banned: int = 4) -> Routing:
    rng = np.random.default_rng(seed)
    ranks = rng.permutation(num_experts) + 1
    p = ranks.astype(np.float64) ** (-zipf_s)
    banned = np.sort(rng.choice(num_experts, size=num_banned, replace=False))
    p[banned] = 0.0
    p /= p.sum()
    logp = np.full(num_experts, -np.inf)
    logp[p > 0] = np.log(p[p > 0])
    chosen = np.empty((num_tokens, top_k), dtype=np.int64)
    chunk = 4096
    for t0 in range(0, num_tokens, chunk):
        t1 = min(num_tokens, t0 + chunk)
        g = rng.gumbel(size=(t1 - t0, num_experts))
        keys = logp[None, :] + g
        top = np.argpartition(-keys, top_k - 1, axis=1)[:, :top_k]
        chosen[t0:t1] = top
    expert = chosen.reshape(-1)
    token = np.repeat(np.arange(num_tokens, dtype=np.int64), top_k)
    order = np.lexsort((token, expert))
    counts = np.bincount(expert, minlength=num_experts).astype(np.int64)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    return Routing(offsets=offsets.astype(np.int32), token_of_row=token[order], counts=counts,
                   banned=banned)


# --- workloads ------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "fprop" | "dgrad" | "wgrad" | "moe"
    M: int
    N: int
    K: int
    in_dtype: str      # "f32" | "bf16"
    out_dtype: str     # "bf16" | "f32"


TINY = Workload("dense-fprop-256x256x512", "fprop", 256, 256, 512, "f32", "bf16")
FPROP = Workload("dense-fprop-8192x18432x7168", "fprop", 8192, 18432, 7168, "bf16", "bf16")
DGRAD = Workload("dgrad-8192x7168x18432", "dgrad", 8192, 7168, 18432, "bf16", "f32")
WGRAD = Workload("wgrad-2048x7168x8192", "wgrad", 2048, 7168, 8192, "bf16", "f32")
MOE = Workload("moe-fprop-256e-32768tok-top8-2048x7168", "moe", 262144, 2048, 7168, "bf16",
               "bf16")
MOE_EXPERTS, MOE_TOKENS, MOE_TOPK, MOE_ZIPF = 256, 32768, 8, 1.1


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def tiny_inputs():
    """A[256,512] fp32 N(0,1) with 0.1% outliers x100; W[256,512] fp32 N(0,0.02)."""
    a = normal_with_outliers((256, 512), 1.0, 101, 0.001, 100.0)
    w = normal_f32((256, 512), 0.02, 102)
    return a, w


def fprop_inputs(m=8192, n=18432, k=7168):
    """A[M,K] bf16 N(0,1) with 0.1% outliers x50; W[N,K] bf16 N(0,0.02)."""
    a = f32_to_bf16_bits(normal_with_outliers((m, k), 1.0, 201, 0.001, 50.0))
    w = f32_to_bf16_bits(normal_f32((n, k), 0.02, 202))
    return a, w


def dgrad_inputs(m=8192, n=18432, k=7168):
    """dY[M,N] bf16 N(0,1e-3); W[N,K] as for the forward pass."""
    dy = f32_to_bf16_bits(normal_f32((m, n), 1e-3, 301))
    w = f32_to_bf16_bits(normal_f32((n, k), 0.02, 202))
    return dy, w


def wgrad_inputs(t=8192, n=2048, k=7168):
    """dY[T,N] and X[T,K], bf16 N(0,1)."""
    dy = f32_to_bf16_bits(normal_f32((t, n), 1.0, 401))
    x = f32_to_bf16_bits(normal_f32((t, k), 1.0, 402))
    return dy, x


def moe_routing_default() -> Routing:
    return moe_routing(MOE_EXPERTS, MOE_TOKENS, MOE_TOPK, MOE_ZIPF, 500)


def moe_tokens(num_tokens=MOE_TOKENS, k=7168) -> np.ndarray:
    """X_tok[T,K] bf16 N(0,1); grouped rows are X_tok[token_of_row]."""
    return f32_to_bf16_bits(normal_f32((num_tokens, k), 1.0, 501))


def moe_expert_weight(e: int, n=2048, k=7168) -> np.ndarray:
    """W_e[N,K] bf16 N(0,0.02), seed 5000+e."""
    return f32_to_bf16_bits(normal_f32((n, k), 0.02, 5000 + e))


def moe_expert_weights(experts, n=2048, k=7168, out: np.ndarray | None = None,
                       workers: int | None = None) -> np.ndarray:
    """Stack of W_e for the listed experts, drawn in parallel threads."""
    experts = list(experts)
    if out is None:
        out = np.empty((len(experts), n, k), dtype=np.uint16)
    workers = workers or min(16, len(os.sched_getaffinity(0)))

    def fill(i):
        out[i] = moe_expert_weight(experts[i], n, k)

    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, range(len(experts))))
    return out


# --- seeded output samples --------------------------------------------------------
# Which output elements the large configurations are checked (and the CPU
# baseline is timed) on: row and column indices only, no arithmetic.

def output_sample(M: int, N: int, seed: int, rows: int = 64, cols: int = 64, rand: int = 4096,
                  block: int = 128):
    """`rows` full rows, `cols` full columns, `rand` random elements and every
    element of the first and last block x block output tiles (which carry the
    M and N tails), seeded; returns (mi, ni) sorted row-major, no repeats."""
    rng = np.random.default_rng(seed)
    ms, ns = [], []
    for m in rng.choice(M, size=min(rows, M), replace=False):
        ms.append(np.full(N, m))
        ns.append(np.arange(N))
    for n in rng.choice(N, size=min(cols, N), replace=False):
        ms.append(np.arange(M))
        ns.append(np.full(M, n))
    ms.append(rng.integers(0, M, rand))
    ns.append(rng.integers(0, N, rand))
    for m0, n0 in ((0, 0), ((M - 1) // block * block, (N - 1) // block * block)):
        mm, nn = np.meshgrid(np.arange(m0, min(M, m0 + block)), np.arange(n0, min(N, n0 + block)),
                             indexing="ij")
        ms.append(mm.ravel())
        ns.append(nn.ravel())
    mi = np.concatenate(ms).astype(np.int64)
    ni = np.concatenate(ns).astype(np.int64)
    key = np.unique(mi * N + ni)
    return key // N, key % N


def expert_rows(offsets: np.ndarray, seed: int, per: int = 8) -> np.ndarray:
    """For every non-empty group of rows [offsets[e], offsets[e+1]): its first
    and last row and `per` distinct random rows (all of them when fewer),
    seeded; sorted, no repeats."""
    rng = np.random.default_rng(seed)
    rows = []
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        rows += [r0, r1 - 1]
        rows += list(r0 + rng.choice(r1 - r0, size=min(per, r1 - r0), replace=False))
    return np.unique(np.array(rows, dtype=np.int64))
