"""Seeded synthetic inputs for the FP8 weight-only linear layer.

This module only draws random numbers and casts the activations and biases to
their activation dtype (torch's round-to-nearest-even cast, which is how a model
would hand them over). It holds none of the method's arithmetic, so both the
CPU oracle and the HIP path can take their inputs from here.

Every tensor comes from numpy's PCG64 seeded with
``SeedSequence([0xF8, workload_id, tensor_id, sub_id])`` so a draw never depends on
the order in which other tensors were drawn. tensor_id: 0 weight, 1 bias,
2 activations, 3 row selection, 4 activation-outlier selection.

Workloads (weights are nn.Linear-shaped [N out, K in], all fp32 before
quantization; activations are [M, K]):

1. tiny GEMV: W [1024,1024] ~ N(0, 0.02^2); bias ~ N(0, 0.01^2) in bf16;
   x [1,1024] bf16 ~ N(0,1).
2. decode GEMV, M=1: W [4096,4096], [14336,4096], [4096,14336] ~ N(0, 0.02^2);
   x [1,K] bf16 ~ N(0,1); bias all zeros (bf16).
3. skinny sweep: W [14336,4096] = 0.02 * Student-t(3); bias ~ N(0, 0.01^2) in
   fp16; x [M,4096] fp16 ~ N(0,1) for M in 2,4,8,16,22,32.
4. decoder block at M=16, bf16: q,k,v,o [4096,4096], gate,up [14336,4096],
   down [4096,14336]; W ~ N(0, 0.02^2); a seeded permutation scales the first
   round(0.01 N) rows by 50 (outlier channels) and sets the next
   round(0.005 N) rows to zero; no bias.
5. large sweep: W [28672,8192], [8192,28672] and [28672,8200] ~ N(0, 0.015^2);
   x [M,K] bf16 ~ N(0,1) with 0.1 % of entries (seeded) multiplied by 20;
   no bias; M in 1,4,8,32.

Prefill, W8A8 (workload id 7): the decoder block's three distinct shapes q
[4096,4096], gate [14336,4096] and down [4096,14336], W ~ N(0, 0.02^2), no bias;
x [M,K] bf16 ~ N(0,1) with 0.1 % of entries (seeded) multiplied by 20, for M
in 512, 2048, 4096 (batches far above the weight-only kernels' 32 tokens).

Batched decode (workload id 8): the decode workload's three weights (workload 2)
at M = 64, 128, 256 tokens; x [M,K] bf16 ~ N(0,1); bias all zeros (bf16), as
in decode. Above the skinny kernels' 32 tokens and below prefill sizes.

Context shape (workload id 6): the one timing of this method the pages print is
for x [22,1024] times a [1024,4096] weight ("FP8 weight-only (precision:
fp8_weights)", the Triton variant in "Dequantise in registers"); it is drawn
like the decode workload: W [4096,1024] ~ N(0, 0.02^2), x [22,1024] bf16 ~
N(0,1), no bias.
"""
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

W_ID, BIAS_ID, X_ID, ROWSEL_ID, XOUT_ID = 0, 1, 2, 3, 4

DECODER_BLOCK = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
                 ("o", 4096, 4096), ("gate", 14336, 4096), ("up", 14336, 4096),
                 ("down", 4096, 14336)]
DECODE_SHAPES = [(4096, 4096), (14336, 4096), (4096, 14336)]
SKINNY_MS = [2, 4, 8, 16, 22, 32]
LARGE_SHAPES = [(28672, 8192), (8192, 28672)]
LARGE_FALLBACK_SHAPE = (28672, 8200)
LARGE_MS = [1, 4, 8, 32]
PAGES_EXAMPLE = (22, 4096, 1024)  # m, n, k
PREFILL_SHAPES = [(4096, 4096), (14336, 4096), (4096, 14336)]
PREFILL_MS = [512, 2048, 4096]
BATCH_MS = [64, 128, 256]
# the decoder block with the layers that share an input merged into one call:
# q/k/v, o, gate/up, down (indices into DECODER_BLOCK)
MERGED_BLOCK = [(0, 1, 2), (3,), (4, 5), (6,)]


def rng(workload: int, tensor: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0xF8, workload, tensor, sub])))


def normal_f32(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def to_act(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """fp32 array -> CPU tensor of the activation dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


@dataclass
class Linear:
    """One linear layer's inputs: fp32 weight, activation-dtype bias (or None)."""
    name: str
    w: np.ndarray
    bias: Optional[torch.Tensor]


@dataclass
class Case:
    """One call: a layer plus its activation block x [M, K] (CPU, activation dtype)."""
    layer: Linear
    x: torch.Tensor


def weight_normal(workload: int, sub: int, n: int, k: int, std: float) -> np.ndarray:
    return normal_f32(rng(workload, W_ID, sub), (n, k), std)


def activations(workload: int, sub: int, m: int, k: int, dtype: torch.dtype,
                outlier_frac: float = 0.0, outlier_gain: float = 20.0) -> torch.Tensor:
    x = normal_f32(rng(workload, X_ID, sub), (m, k), 1.0)
    if outlier_frac > 0.0:
        cnt = int(round(outlier_frac * m * k))
        idx = rng(workload, XOUT_ID, sub).choice(m * k, size=cnt, replace=False)
        flat = x.reshape(-1)
        flat[idx] *= np.float32(outlier_gain)
    return to_act(x, dtype)


# ------------------------------------------------------------------ workloads
def tiny_gemv():
    w = weight_normal(1, 0, 1024, 1024, 0.02)
    bias = to_act(normal_f32(rng(1, BIAS_ID), (1024,), 0.01), torch.bfloat16)
    x = activations(1, 0, 1, 1024, torch.bfloat16)
    return Case(Linear("tiny", w, bias), x)


def decode_layer(i: int) -> Linear:
    n, k = DECODE_SHAPES[i]
    w = weight_normal(2, i, n, k, 0.02)
    return Linear(f"decode_{n}x{k}", w, torch.zeros(n, dtype=torch.bfloat16))


def decode_x(i: int) -> torch.Tensor:
    n, k = DECODE_SHAPES[i]
    return activations(2, i, 1, k, torch.bfloat16)


def skinny_layer() -> Linear:
    g = rng(3, W_ID)
    w = (g.standard_t(3.0, size=(14336, 4096)) * 0.02).astype(np.float32)
    bias = to_act(normal_f32(rng(3, BIAS_ID), (14336,), 0.01), torch.float16)
    return Linear("skinny_14336x4096", w, bias)


def skinny_x(m: int) -> torch.Tensor:
    return activations(3, m, m, 4096, torch.float16)


def block_layer(i: int) -> Linear:
    name, n, k = DECODER_BLOCK[i]
    w = weight_normal(4, i, n, k, 0.02)
    perm = rng(4, ROWSEL_ID, i).permutation(n)
    n_out = int(round(0.01 * n))
    n_zero = int(round(0.005 * n))
    w[perm[:n_out]] *= np.float32(50.0)
    w[perm[n_out:n_out + n_zero]] = 0.0
    return Linear(name, w, None)


def block_x(i: int) -> torch.Tensor:
    _, n, k = DECODER_BLOCK[i]
    return activations(4, i, 16, k, torch.bfloat16)


def large_layer(shape) -> Linear:
    n, k = shape
    sub = {(28672, 8192): 0, (8192, 28672): 1, (28672, 8200): 2}[(n, k)]
    return Linear(f"large_{n}x{k}", weight_normal(5, sub, n, k, 0.015), None)


def large_x(shape, m: int) -> torch.Tensor:
    n, k = shape
    sub = {(28672, 8192): 0, (8192, 28672): 1, (28672, 8200): 2}[(n, k)]
    return activations(5, 100 * sub + m, m, k, torch.bfloat16, outlier_frac=0.001)


def batch_x(i: int, m: int) -> torch.Tensor:
    n, k = DECODE_SHAPES[i]
    return activations(8, 1000 * i + m, m, k, torch.bfloat16)


def prefill_layer(i: int) -> Linear:
    n, k = PREFILL_SHAPES[i]
    return Linear(f"prefill_{n}x{k}", weight_normal(7, i, n, k, 0.02), None)


def prefill_x(i: int, m: int) -> torch.Tensor:
    n, k = PREFILL_SHAPES[i]
    return activations(7, 10000 * i + m, m, k, torch.bfloat16, outlier_frac=0.001)


def pages_example():
    m, n, k = PAGES_EXAMPLE
    return Case(Linear(f"example_{n}x{k}", weight_normal(6, 0, n, k, 0.02), None),
                activations(6, 0, m, k, torch.bfloat16))


# ------------------------------------------------------------------ small parity cases
def random_case(seed: int, m: int, n: int, k: int, dtype: torch.dtype, with_bias: bool = True,
                std: float = 0.02) -> Case:
    """A small seeded case of any shape (used by parity tests at tile/tail sizes)."""
    w = normal_f32(rng(100 + seed, W_ID), (n, k), std)
    bias = to_act(normal_f32(rng(100 + seed, BIAS_ID), (n,), 0.01), dtype) if with_bias else None
    x = activations(100 + seed, 0, m, k, dtype)
    return Case(Linear(f"rand{seed}_{n}x{k}", w, bias), x)


def all_workload_names() -> List[str]:
    return ["tiny_gemv", "decode", "skinny", "decoder_block", "large", "prefill"]
