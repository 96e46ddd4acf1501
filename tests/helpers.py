"""Shared helpers for the GPU parity tests: host <-> device marshalling, the
seeded output-element samples, and the comparison against the oracle."""
from __future__ import annotations

import numpy as np
import torch


def to_dev(x: np.ndarray, dev="cuda") -> torch.Tensor:
    """float32 arrays become float32 tensors; uint16 arrays are BF16 bits."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def codes(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def scale_bits(t: torch.Tensor) -> np.ndarray:
    return np.ascontiguousarray(t.cpu().numpy()).view(np.uint32)


def assert_same_bytes(gpu: np.ndarray, ref: np.ndarray, what: str):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if not np.array_equal(gpu, ref):
        bad = np.argwhere(gpu != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: gpu {gpu[i]!r} "
                             f"oracle {ref[i]!r}")


def sample_elements(M: int, N: int, seed: int, rows: int = 64, cols: int = 64,
                    rand: int = 4096, block: int = 128):
    """Seeded output sample: `rows` full rows, `cols` full columns, `rand`
    random elements, and every element of the first and last block x block
    output tiles (which carry the M and N tails)."""
    from fp8_fine_grained_quant_amd import synth
    return synth.output_sample(M, N, seed, rows, cols, rand, block)


def per_tile_elements(m_starts, m_ends, N: int, seed: int, per: int = 4, tile_m: int = 256,
                      tile_n: int = 256):
    """`per` seeded random elements inside every output tile: rows are cut
    into tiles of tile_m from each start in m_starts up to the matching end
    (one start/end pair per group; a dense GEMM is one group), columns into
    tiles of tile_n."""
    rng = np.random.default_rng(seed)
    ms, ns = [], []
    for m0, m1 in zip(m_starts, m_ends):
        for r0 in range(int(m0), int(m1), tile_m):
            r1 = min(int(m1), r0 + tile_m)
            for c0 in range(0, N, tile_n):
                c1 = min(N, c0 + tile_n)
                ms.append(rng.integers(r0, r1, per))
                ns.append(rng.integers(c0, c1, per))
    if not ms:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(ms).astype(np.int64), np.concatenate(ns).astype(np.int64)


def union_elements(N: int, *pairs):
    """Union of (mi, ni) element lists, sorted row-major without repeats."""
    key = np.unique(np.concatenate([np.asarray(m, np.int64) * N + np.asarray(n, np.int64)
                                    for m, n in pairs]))
    return key // N, key % N


def check_gemm(c_gpu: np.ndarray, c_ref: np.ndarray, s_ref: np.ndarray, bf16_out: bool,
               what: str) -> float:
    """|gpu - C*| <= 1e-3 * S (+ one BF16 ulp of C* for BF16 output), all
    finite.  Returns max |err| / tol (at most 1 when the check passes) over
    elements with a non-zero tolerance."""
    from oracle import oracle
    g = np.asarray(c_gpu, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    tol = oracle.gemm_tolerance(c_ref, s_ref, bf16_out)
    err = np.abs(g - c_ref)
    bad = err > tol
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first flat "
                             f"index {i}: gpu {g.ravel()[i]!r} exact {c_ref.ravel()[i]!r} "
                             f"tol {tol.ravel()[i]!r}")
    rel = err / np.where(tol > 0, tol, np.inf)
    return float(rel.max()) if rel.size else 0.0
