"""One training step of a two-layer perceptron through the fused epilogue plans.

The pages use the fused epilogues this way: RELU_AUX_BIAS in the forward pass keeps
the ReLU mask, and DRELU_BGRAD in the backward pass consumes it and returns the bias
gradient ("Fusing epilogs with matrix multiplication using nvmath-python", sections
on the forward epilogs and on the DRELU_BGRAD path; its FAQ notes that the weight
gradients and the rest of the step come from other products). This module wires the
five products of such a step; each is one execute of a plan of the C ABI, so every
step of the computation runs in the library's kernels. Nothing here computes.

Layout (features along rows, the batch along columns, one bias per row, as the
library's bias convention has it):
  X (d, b); W1 (h, d), b1 (h); W2 (o, h)
  forward:  H  = relu(W1 X + b1)   (h, b)   RELU_AUX_BIAS, mask (ceil(h/32), b)
            Y  = W2 H              (o, b)   NONE
  backward, given dY (o, b):
            dW2 = dY H^T           (o, h)   NONE, B = H as stored (n, k)
            dZ1 = mask * (W2^T dY) (h, b)   DRELU_BGRAD, A = W2 as stored (k, m);
            db1 = sum over the batch of dZ1 (its bias gradient output)
            dW1 = dZ1 X^T          (h, d)   NONE, B = X as stored (n, k)
The input gradient dX = W1^T dZ1 is not formed: X is the network's input.
All sizes must be multiples of 8 (16-bit rows; h because W2 is read transposed).

With fused=False the same step runs the unfused baselines in place of the two fused
epilogues, each step of them its own kernel with its output in memory ("Operator fusion
in AI inference compilers", section 2.2 diagram): the forward's GEMM -> T1, bias add ->
T2, ReLU -> H chain, which keeps H but no mask, and the backward's GEMM -> T1, ReLU
backward against H -> dZ1, row sums -> db1 chain.
"""
from typing import Dict

import torch

from . import Matmul

_TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


class MLP2Step:
    """Plans for one (d, h, o, batch) shape; `forward` and `backward` enqueue on the
    current torch stream and return device tensors (outputs are allocated once and
    reused by every call)."""

    def __init__(self, d: int, h: int, o: int, batch: int, dtype: str = "bf16", fused: bool = True):
        if dtype not in _TORCH:
            raise ValueError("the step runs in fp16 or bf16")
        for name, v in (("d", d), ("h", h), ("o", o), ("batch", batch)):
            if v < 8 or v % 8:
                raise ValueError(f"{name} = {v} must be a positive multiple of 8")
        self.d, self.h, self.o, self.b, self.dtype, self.fused = d, h, o, batch, dtype, bool(fused)
        self.fwd1 = Matmul(h, batch, d, dtype, "RELU_AUX_BIAS" if fused else "RELU_BIAS_UNFUSED")
        self.fwd2 = Matmul(o, batch, h, dtype, "NONE")
        self.dw2 = Matmul(o, h, batch, dtype, "NONE", trans_b=True)
        self.dz1 = Matmul(h, batch, o, dtype, "DRELU_BGRAD" if fused else "DRELU_BGRAD_UNFUSED", trans_a=True)
        self.dw1 = Matmul(h, d, batch, dtype, "NONE", trans_b=True)
        self.plans = (self.fwd1, self.fwd2, self.dw2, self.dz1, self.dw1)
        for p in self.plans:
            p.plan()
        t = _TORCH[dtype]
        dev = torch.device("cuda", torch.cuda.current_device())
        self.H = torch.empty(h, batch, dtype=t, device=dev)
        self.mask = torch.empty((h + 31) // 32, batch, dtype=torch.int32, device=dev) if fused else None
        self.Y = torch.empty(o, batch, dtype=t, device=dev)
        self.dW2 = torch.empty(o, h, dtype=t, device=dev)
        self.dZ1 = torch.empty(h, batch, dtype=t, device=dev)
        self.db1 = torch.empty(h, dtype=t, device=dev)
        self.dW1 = torch.empty(h, d, dtype=t, device=dev)

    def flops(self) -> int:
        """Multiply-adds of the five products, counted as 2 flops each."""
        d, h, o, b = self.d, self.h, self.o, self.b
        return 2 * (h * b * d + o * b * h + o * h * b + h * b * o + h * d * b)

    def forward(self, X, W1, b1, W2) -> torch.Tensor:
        if self.fused:
            self.fwd1.execute(W1, X, b1, relu_aux=self.mask, out=self.H)
        else:
            self.fwd1.execute(W1, X, b1, out=self.H)
        self.fwd2.execute(W2, self.H, out=self.Y)
        return self.Y

    def backward(self, X, W2, dY) -> Dict[str, torch.Tensor]:
        self.dw2.execute(dY, self.H, out=self.dW2)
        if self.fused:
            self.dz1.execute(W2, dY, relu_aux=self.mask, out=self.dZ1, bgrad=self.db1)
        else:
            self.dz1.execute(W2, dY, act=self.H, out=self.dZ1, bgrad=self.db1)
        self.dw1.execute(self.dZ1, X, out=self.dW1)
        return {"dW1": self.dW1, "db1": self.db1, "dW2": self.dW2, "dZ1": self.dZ1}

    def step(self, X, W1, b1, W2, dY) -> Dict[str, torch.Tensor]:
        self.forward(X, W1, b1, W2)
        return self.backward(X, W2, dY)

    def free(self):
        for p in self.plans:
            p.free()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()
        return False
