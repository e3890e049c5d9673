"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers: it holds none of the epilogue arithmetic, so
both the HIP path and the CPU oracle can take their inputs from it.

Every matrix is drawn in blocks of BLOCK_ROWS rows. Block b of tensor `tag` uses its
own torch CPU generator seeded with mix(seed, tag, b), so any set of whole blocks can
be regenerated without drawing the rest (the oracle checks sampled rows of the large
workloads this way). Values are N(0, 1) * std in fp32, then cast to the storage
dtype by torch (round to nearest even).

The workloads follow the shapes and distributions of the pages' examples: the
(m,n,k) = (1024,512,2048) fp16 example of the cuBLASLt-wrapper page, the 7B FFN
layer M=4096, N=11008 of the operator-fusion page, and the (65536,16384)x(16384,8192)
fp16 H200 shape of the nvmath epilog page. "N(0, s)" means standard deviation s.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import torch

BLOCK_ROWS = 256

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# tensor tags (part of the seed)
TAG_A, TAG_B, TAG_BIAS, TAG_A2, TAG_B2 = 1, 2, 3, 4, 5
TAG_X, TAG_W1, TAG_B1, TAG_W2, TAG_DY = 6, 7, 8, 9, 10


def _mix(seed: int, tag: int, block: int) -> int:
    x = (seed * 0x9E3779B1 + tag * 0x85EBCA77 + block * 0xC2B2AE3D) & ((1 << 63) - 1)
    x ^= x >> 29
    x = (x * 0xBF58476D1CE4E5B9) & ((1 << 63) - 1)
    x ^= x >> 32
    return x


def normal(rows: int, cols: int, std: float, dtype: str, seed: int, tag: int,
           r0: int = 0, r1: Optional[int] = None) -> torch.Tensor:
    """Rows [r0, r1) of a (rows, cols) N(0, std) matrix, as a CPU tensor of `dtype`."""
    r1 = rows if r1 is None else r1
    assert 0 <= r0 <= r1 <= rows
    out = torch.empty((r1 - r0, cols), dtype=TORCH_DT[dtype])
    b0, b1 = r0 // BLOCK_ROWS, (r1 + BLOCK_ROWS - 1) // BLOCK_ROWS
    for b in range(b0, b1):
        lo, hi = b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS)
        g = torch.Generator().manual_seed(_mix(seed, tag, b))
        blk = torch.randn((hi - lo, cols), generator=g, dtype=torch.float32)
        blk.mul_(std)
        s0, s1 = max(lo, r0), min(hi, r1)
        out[s0 - r0:s1 - r0] = blk[s0 - lo:s1 - lo].to(TORCH_DT[dtype])
    return out


def vector(length: int, std: float, dtype: str, seed: int, tag: int) -> torch.Tensor:
    return normal(length, 1, std, dtype, seed, tag).reshape(length)


@dataclass
class Workload:
    """One synthetic problem. Forward: D = act(A B + bias). Backward (if any):
    D2 = mask * (A2 B2), bgrad = sum over n, consuming the forward mask."""
    name: str
    m: int
    n: int
    k: int
    dtype: str                   # storage type of A, B and D
    epilog: str                  # forward epilogue
    std_a: float
    std_b: float
    std_bias: float
    vec: Optional[str] = None    # bias / bgrad dtype (defaults to dtype)
    std_a2: Optional[float] = None   # backward operands, when the workload has a backward
    std_b2: Optional[float] = None
    seed: int = 0
    extra: Dict[str, str] = field(default_factory=dict)

    @property
    def vec_dtype(self) -> str:
        return self.vec or self.dtype

    @property
    def has_backward(self) -> bool:
        return self.std_a2 is not None

    def flops(self) -> int:
        return 2 * self.m * self.n * self.k

    def a(self, r0: int = 0, r1: Optional[int] = None) -> torch.Tensor:
        return normal(self.m, self.k, self.std_a, self.dtype, self.seed, TAG_A, r0, r1)

    def b(self) -> torch.Tensor:
        return normal(self.k, self.n, self.std_b, self.dtype, self.seed, TAG_B)

    def bias(self) -> torch.Tensor:
        return vector(self.m, self.std_bias, self.vec_dtype, self.seed, TAG_BIAS)

    def a2(self, r0: int = 0, r1: Optional[int] = None) -> torch.Tensor:
        return normal(self.m, self.k, self.std_a2, self.dtype, self.seed, TAG_A2, r0, r1)

    def b2(self) -> torch.Tensor:
        return normal(self.k, self.n, self.std_b2, self.dtype, self.seed, TAG_B2)


def _w(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    # tiny fp32 MLP step: RELU_AUX_BIAS forward, then DRELU_BGRAD on fresh operands
    _w(name="mlp_tiny_f32_64x48x32", m=64, n=48, k=32, dtype="f32", epilog="RELU_AUX_BIAS",
       std_a=1.0, std_b=1.0, std_bias=0.1, std_a2=1.0, std_b2=1.0),
    # the cuBLASLt-wrapper page's PyTorch example
    _w(name="relu_bias_f16_1024x512x2048", m=1024, n=512, k=2048, dtype="f16", epilog="RELU_BIAS",
       std_a=1.0, std_b=1.0, std_bias=1.0),
    # 7B FFN layer, fused RELU_BIAS (the headline workload) and its bf16 GELU_BIAS twin
    _w(name="ffn_f16_4096x11008x4096", m=4096, n=11008, k=4096, dtype="f16", epilog="RELU_BIAS",
       std_a=1.0 / 64, std_b=1.0 / 64, std_bias=0.02),
    _w(name="ffn_gelu_bf16_4096x11008x4096", m=4096, n=11008, k=4096, dtype="bf16", epilog="GELU_BIAS",
       std_a=1.0 / 64, std_b=1.0 / 64, std_bias=0.02),
    # 2-layer MLP training pair, batch 8192, hidden 8192
    _w(name="mlp_bf16_8192", m=8192, n=8192, k=8192, dtype="bf16", epilog="RELU_AUX_BIAS",
       std_a=8192 ** -0.5, std_b=1.0, std_bias=0.02, std_a2=8192 ** -0.5, std_b2=1.0),
    # one GPU's share of an 8-way split along n (the batch columns of B and D): the FFN
    # layer with n = 11008 / 8, and the 8192 MLP pair with n = 8192 / 8; and of a 4-way
    # split of the FFN layer, n = 11008 / 4
    _w(name="ffn_shard8_f16_4096x1376x4096", m=4096, n=1376, k=4096, dtype="f16", epilog="RELU_BIAS",
       std_a=1.0 / 64, std_b=1.0 / 64, std_bias=0.02),
    _w(name="ffn_shard4_f16_4096x2752x4096", m=4096, n=2752, k=4096, dtype="f16", epilog="RELU_BIAS",
       std_a=1.0 / 64, std_b=1.0 / 64, std_bias=0.02),
    _w(name="mlp_shard8_bf16_8192x1024x8192", m=8192, n=1024, k=8192, dtype="bf16", epilog="RELU_AUX_BIAS",
       std_a=8192 ** -0.5, std_b=1.0, std_bias=0.02, std_a2=8192 ** -0.5, std_b2=1.0),
    # the square benchmark size the epilog-configuration page recommends for comparing
    # fused and unfused latency (distributions as for the FFN layer)
    _w(name="square_f16_4096", m=4096, n=4096, k=4096, dtype="f16", epilog="RELU_BIAS",
       std_a=1.0 / 64, std_b=1.0 / 64, std_bias=0.02),
    # the H200 comparison shape, RELU_BIAS and (same inputs) RELU_AUX_BIAS
    _w(name="large_f16_65536x8192x16384", m=65536, n=8192, k=16384, dtype="f16", epilog="RELU_BIAS",
       std_a=1.0 / 128, std_b=1.0 / 128, std_bias=0.02),
]}

HEADLINE = "ffn_f16_4096x11008x4096"


def small_case(m: int, n: int, k: int, dtype: str, std: float = 1.0, std_bias: float = 1.0,
               seed: int = 0, vec: Optional[str] = None) -> Tuple[torch.Tensor, ...]:
    """A, B, bias and backward A2, B2 for an arbitrary small shape."""
    v = vec or dtype
    return (normal(m, k, std, dtype, seed, TAG_A), normal(k, n, std, dtype, seed, TAG_B),
            vector(m, std_bias, v, seed, TAG_BIAS), normal(m, k, std, dtype, seed, TAG_A2),
            normal(k, n, std, dtype, seed, TAG_B2))


def mlp_case(d: int, h: int, o: int, batch: int, dtype: str, seed: int = 0) -> Tuple[torch.Tensor, ...]:
    """X (d, batch) ~ N(0,1), W1 (h, d) ~ N(0, 1/sqrt(d)), b1 (h) ~ N(0, 0.02),
    W2 (o, h) ~ N(0, 1/sqrt(h)) and the output gradient dY (o, batch) ~ N(0,1) of a
    two-layer perceptron step (features along rows, the batch along columns)."""
    return (normal(d, batch, 1.0, dtype, seed, TAG_X), normal(h, d, d ** -0.5, dtype, seed, TAG_W1),
            vector(h, 0.02, dtype, seed, TAG_B1), normal(o, h, h ** -0.5, dtype, seed, TAG_W2),
            normal(o, batch, 1.0, dtype, seed, TAG_DY))


def integer_case(m: int, n: int, k: int, dtype: str, seed: int = 0, vec: Optional[str] = None,
                 second: bool = True):
    """Integer-valued A, B in [-2, 2] and half-integer bias in [-7.5, 7.5].

    With k <= 16 every product, sum and biased value is exact in fp32, fp16 and bf16,
    and no pre-activation is zero, so any correct implementation gives the same bits.
    (For any k below 2^21 the fp32 sums and biased values stay exact, so the same holds up to
    the one rounding of the output, which both sides take alike.) second = False
    leaves out the second pair of operands (A2, B2 are then None); the first draws
    are the same either way.
    """
    v = vec or dtype
    g = torch.Generator().manual_seed(_mix(seed, 99, m * 131 + n * 17 + k))
    A = torch.randint(-2, 3, (m, k), generator=g).to(TORCH_DT[dtype])
    B = torch.randint(-2, 3, (k, n), generator=g).to(TORCH_DT[dtype])
    bias = (torch.randint(-8, 8, (m,), generator=g).to(torch.float32) + 0.5).to(TORCH_DT[v])
    if not second:
        return A, B, bias, None, None
    A2 = torch.randint(-2, 3, (m, k), generator=g).to(TORCH_DT[dtype])
    B2 = torch.randint(-2, 3, (k, n), generator=g).to(TORCH_DT[dtype])
    return A, B, bias, A2, B2


def integer_tie_case(m: int, n: int, k: int, dtype: str, seed: int = 0, vec: Optional[str] = None):
    """As integer_case, but with an integer bias in [-8, 8]: pre-activations are
    integers, and a share of them is exactly 0 (the ReLU tie)."""
    v = vec or dtype
    g = torch.Generator().manual_seed(_mix(seed, 98, m * 131 + n * 17 + k))
    A = torch.randint(-2, 3, (m, k), generator=g).to(TORCH_DT[dtype])
    B = torch.randint(-2, 3, (k, n), generator=g).to(TORCH_DT[dtype])
    bias = torch.randint(-8, 9, (m,), generator=g).to(torch.float32).to(TORCH_DT[v])
    A2 = torch.randint(-2, 3, (m, k), generator=g).to(TORCH_DT[dtype])
    B2 = torch.randint(-2, 3, (k, n), generator=g).to(TORCH_DT[dtype])
    return A, B, bias, A2, B2
