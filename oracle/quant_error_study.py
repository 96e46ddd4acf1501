"""Quantization-error study on the CPU oracle (analysis only, no GPU).

TEST / ANALYSIS INFRASTRUCTURE: this script runs only the CPU oracle and
numpy.  The product library never imports it.

It measures what fine-grained scaling buys on the synthetic workloads.  The
pages motivate tile- and block-wise scaling by activation outliers, which
make one max-abs scale per tensor waste the FP8 range on every other value
("Should Fixing Deepseek Take 60 Steps?", mixed-precision framework passage;
Figure 7(a)).  They also choose E4M3 over E5M2 for all tensors, gradients
included, because fine-grained scaling makes the extra mantissa bit usable
(jp-study.kr page, E4M3-on-all-tensors passage).

For each tensor and scaling scheme the study reports:
  * tensor error: ||x - dequant(quant(x))|| / ||x|| (Frobenius, fp64);
  * GEMM error: ||C - C_q|| / ||C|| where C is the fp64 product of the
    unquantized inputs and C_q the fp64 product of the dequantized operands
    (equal, up to fp64 rounding, to the exact block-scaled GEMM).
Schemes: one scale per tensor; one per row (1 x K); the method's 1x128 /
128x128 groups; and, for gradients, E5M2 in place of E4M3.  E4M3 uses the
oracle's encoder and scale rule; E5M2 (largest finite 57344) uses PyTorch's
CPU float8_e5m2 cast, which rounds to nearest even, on values pre-scaled
into range.

Usage: python oracle/quant_error_study.py [--rows 1024] [--wrows 2048]
Prints a markdown table.
"""
from __future__ import annotations

import argparse
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path[:] = [ROOT] + [q for q in sys.path if os.path.abspath(q or ".") != os.path.dirname(
    os.path.abspath(__file__))]

from oracle import oracle  # noqa: E402
from fp8_fine_grained_quant_amd import synth  # noqa: E402

E5M2_MAX = 57344.0


def e4m3_groups(x32: np.ndarray, gr: int, gc: int) -> np.ndarray:
    """Dequantized E4M3 values with one scale per gr x gc group (the
    oracle's scale rule and encoder; gr/gc = 0 means the whole extent)."""
    R, C = x32.shape
    gr, gc = gr or R, gc or C
    out = np.empty((R, C), dtype=np.float64)
    for r0 in range(0, R, gr):
        for c0 in range(0, C, gc):
            blk = x32[r0:r0 + gr, c0:c0 + gc]
            s, inv = oracle.group_scale(float(np.max(np.abs(blk))))
            q = oracle.e4m3_encode((blk * inv).astype(np.float32))
            out[r0:r0 + gr, c0:c0 + gc] = oracle.e4m3_decode(q) * np.float64(s)
    return out


def e4m3_rows_fast(x32: np.ndarray, gc: int) -> np.ndarray:
    """1 x gc groups through the oracle's own 1x128 quantizer when gc == 128."""
    if gc == 128:
        q, s = oracle.quant_1x128(x32)
        return oracle.e4m3_decode(q) * np.repeat(s.T.astype(np.float64), 128, axis=1)[:, :x32.shape[1]]
    return e4m3_groups(x32, 1, gc)


def e4m3_pow2(x32: np.ndarray, block: bool) -> np.ndarray:
    """The method's groups with power-of-two (E8M0) scales (oracle rule)."""
    if block:
        q, s, _ = oracle.quant_128x128(x32, rule=oracle.RULE_POW2)
        sc = np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)
        return oracle.e4m3_decode(q) * sc[:x32.shape[0], :x32.shape[1]]
    q, s = oracle.quant_1x128(x32, rule=oracle.RULE_POW2)
    return oracle.e4m3_decode(q) * np.repeat(s.T.astype(np.float64), 128, axis=1)[:, :x32.shape[1]]


def e5m2_groups(x32: np.ndarray, gr: int, gc: int) -> np.ndarray:
    import torch
    R, C = x32.shape
    gr, gc = gr or R, gc or C
    out = np.empty((R, C), dtype=np.float64)
    for r0 in range(0, R, gr):
        for c0 in range(0, C, gc):
            blk = x32[r0:r0 + gr, c0:c0 + gc].astype(np.float64)
            amax = np.max(np.abs(blk))
            s = amax / E5M2_MAX if amax > 0 else 1.0
            v = torch.from_numpy((blk / s).astype(np.float32)).to(torch.float8_e5m2).float().numpy()
            out[r0:r0 + gr, c0:c0 + gc] = v.astype(np.float64) * s
    return out


def rel(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def row_p95(a: np.ndarray, b: np.ndarray) -> float:
    """95th percentile over rows of each row's own relative error."""
    return float(np.percentile(np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1), 95))


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--rows", type=int, default=1024, help="activation / gradient rows used")
    p.add_argument("--wrows", type=int, default=2048, help="weight rows used")
    args = p.parse_args()
    R, WR = args.rows, args.wrows

    a_bits, w_bits = synth.fprop_inputs()
    dy_bits, _ = synth.dgrad_inputs()
    a32 = synth.bf16_bits_to_f32(a_bits[:R])
    w32 = synth.bf16_bits_to_f32(w_bits[:WR])
    dy32 = synth.bf16_bits_to_f32(dy_bits[:R, :WR])          # dY[:, :WR] pairs with W[:WR]
    a, w, dy = a32.astype(np.float64), w32.astype(np.float64), dy32.astype(np.float64)
    c_f = a @ w.T                                               # Fprop: A W^T
    c_d = dy @ w                                                # Dgrad: dY W

    acts = {"per-tensor E4M3": e4m3_groups(a32, 0, 0),
            "per-row (1xK) E4M3": e4m3_groups(a32, 1, 0),
            "1x128 E4M3 (method)": e4m3_rows_fast(a32, 128),
            "1x128 E4M3, power-of-two scales": e4m3_pow2(a32, False)}
    # a harder activation: the same values with per-token magnitudes spread
    # over e^[-4, 4] (seeded), as between tokens of different norm
    spread = np.exp(np.random.default_rng(11).uniform(-4.0, 4.0, (R, 1))).astype(np.float32)
    as32 = (a32 * spread).astype(np.float32)
    as64 = as32.astype(np.float64)
    cs_f = as64 @ w.T
    acts_s = {"per-tensor E4M3": e4m3_groups(as32, 0, 0),
              "per-row (1xK) E4M3": e4m3_groups(as32, 1, 0),
              "1x128 E4M3 (method)": e4m3_rows_fast(as32, 128)}
    wts = {"per-tensor E4M3": e4m3_groups(w32, 0, 0),
           "128x128 E4M3 (method)": e4m3_groups(w32, 128, 128),
           "128x128 E4M3, power-of-two scales": e4m3_pow2(w32, True)}
    grads = {"per-tensor E4M3": e4m3_groups(dy32, 0, 0),
             "per-tensor E5M2": e5m2_groups(dy32, 0, 0),
             "1x128 E4M3 (method)": e4m3_rows_fast(dy32, 128),
             "1x128 E5M2": e5m2_groups(dy32, 1, 128)}

    print(f"# fine-grained FP8 quantization error (CPU oracle; A[{R},7168] with 0.1% outliers x50, "
          f"W[{WR},7168] N(0,0.02), dY[{R},{WR}] N(0,1e-3); bf16 inputs)")
    print("| tensor | scheme | tensor rel. error | per-row rel. error, p95 | GEMM rel. error |")
    print("|---|---|---|---|---|")
    wq = wts["128x128 E4M3 (method)"]
    aq = acts["1x128 E4M3 (method)"]
    for k, v in acts.items():
        print(f"| A (Fprop) | {k} | {rel(v, a):.3e} | {row_p95(v, a):.3e} | "
              f"{rel(v @ wq.T, c_f):.3e} (W 128x128) |")
    for k, v in acts_s.items():
        print(f"| A, token norms spread e^[-4,4] | {k} | {rel(v, as64):.3e} | "
              f"{row_p95(v, as64):.3e} | {row_p95(v @ wq.T, cs_f):.3e} (W 128x128; per-row p95) |")
    for k, v in wts.items():
        print(f"| W | {k} | {rel(v, w):.3e} | {row_p95(v, w):.3e} | {rel(aq @ v.T, c_f):.3e} (A 1x128) |")
    for k, v in grads.items():
        print(f"| dY (Dgrad) | {k} | {rel(v, dy):.3e} | {row_p95(v, dy):.3e} | "
              f"{rel(v @ wq, c_d):.3e} (W 128x128) |")
    both = rel(acts["per-tensor E4M3"] @ wts["per-tensor E4M3"].T, c_f)
    print(f"| A, W | both per-tensor E4M3 | | | {both:.3e} |")
    print(f"| A, W | 1x128 / 128x128 (method) | | | {rel(aq @ wq.T, c_f):.3e} |")
    p2 = rel(acts["1x128 E4M3, power-of-two scales"] @ wts["128x128 E4M3, power-of-two scales"].T, c_f)
    print(f"| A, W | 1x128 / 128x128, power-of-two scales | | | {p2:.3e} |")


if __name__ == "__main__":
    main()
