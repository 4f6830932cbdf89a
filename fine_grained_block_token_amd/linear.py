"""One FP8 nn.Linear step (forward, dgrad, wgrad) composed from the library's entry points.

The composition follows the maintainers' reply in "[Help] Starter script for nn.Linear
for fwd,bwd" and "DeepGEMM Essentials", Part 18:

* forward  y  = x W^T:  x cast per token (1 x g groups along the input features), W cast
  per 128 x 128 block, one NT GEMM with bf16 output;
* dgrad    dX = dY W:   dY cast per token, the NT GEMM against the exact FP8 transpose of
  W (and of its block-scale grid) that the block cast emits beside W;
* wgrad    dW += dY^T x: both transposed views cast per token along the tokens (groups of
  128 tokens), the fp32 weight-gradient GEMM accumulating into dW ("DeepGEMM Essentials",
  Parts 12-13).

x and dY are each read once: the dual-orientation cast writes the row-wise operand and
the transposed one from the same read.  Every call below only launches library kernels
on the current stream; the class owns the preallocated FP8 operands, scales and outputs
of one shape.

Recipes:

* ``"fp32"``: fp32 scales (1 x 128 per token, 128 x 128 per block), promoted in fp32;
* ``"ue8m0"``: the same groups with power-of-two scales (stored as fp32 2^e), applied by
  the scaled MFMA without promotion;
* ``"ue8m0_g32"``: 1 x 32 groups with packed UE8M0 scales on every operand (W too is cast
  per 1 x 32 group in both orientations), the GEMMs on the scaled MFMA.
"""
from __future__ import annotations

import torch

from . import (SF_FP32, SF_PACKED_UE8M0, SF_UE8M0, Fgfp8Error, cast_per_block, cast_per_token_dual,
               gemm_fp8_nt_bf16, gemm_fp8_nt_bf16_ue8m0, gemm_fp8_nt_bf16_ue8m0_g32, mn_major_scales,
               wgrad_gemm_fp8_nt_fp32, wgrad_gemm_fp8_nt_fp32_ue8m0, wgrad_gemm_fp8_nt_fp32_ue8m0_g32)

RECIPES = ("fp32", "ue8m0", "ue8m0_g32")


class Fp8Linear:
    """Buffers and launches of one FP8 linear step at a fixed shape: ``x`` [tokens, d_in],
    ``W`` [d_out, d_in], ``dY`` [tokens, d_out] (bf16 or fp32, row-major, on the GPU).

    Outputs: ``y`` [tokens, d_out] bf16, ``dX`` [tokens, d_in] bf16, and ``dW`` [d_out, d_in]
    fp32, which ``backward_weight`` accumulates into (zero it, or leave the previous
    gradient there).  FP8 operands and their scales stay available as attributes:
    ``xq/sx``, ``xTq/sxT``, ``Wq/sW``, ``WqT/sWT``, ``dYq/sdY``, ``dYTq/sdYT``."""

    def __init__(self, tokens: int, d_in: int, d_out: int, recipe: str = "fp32", device="cuda"):
        if recipe not in RECIPES:
            raise Fgfp8Error(f"recipe must be one of {RECIPES}, got {recipe!r}")
        for name, v in (("tokens", tokens), ("d_in", d_in), ("d_out", d_out)):
            # every one of them is a GEMM's K somewhere in the step, and K is a whole
            # number of 128-wide blocks
            if v <= 0 or v % 128:
                raise Fgfp8Error(f"{name} = {v} must be a positive multiple of 128")
        self.T, self.I, self.O, self.recipe = tokens, d_in, d_out, recipe
        T, I, O = tokens, d_in, d_out
        u8, f32 = torch.uint8, torch.float32
        mk = lambda r, c: torch.empty((r, c), dtype=u8, device=device)
        self.xq, self.xTq = mk(T, I), mk(I, T)
        self.Wq, self.WqT = mk(O, I), mk(I, O)
        self.dYq, self.dYTq = mk(T, O), mk(O, T)
        if recipe == "ue8m0_g32":
            # packed words: one int32 per row and 128-wide K block (four 1 x 32 groups)
            w = lambda r, c: mn_major_scales(r, c // 128, torch.int32, device)
            self.sx, self.sxT, self.sW, self.sWT = w(T, I), w(I, T), w(O, I), w(I, O)
            self.sdY, self.sdYT = w(T, O), w(O, T)
        else:
            s = lambda r, c: mn_major_scales(r, c // 128, f32, device)
            self.sx, self.sxT, self.sdY, self.sdYT = s(T, I), s(I, T), s(T, O), s(O, T)
            self.sW = torch.empty((O // 128, I // 128), dtype=f32, device=device)
            self.sWT = torch.empty((I // 128, O // 128), dtype=f32, device=device)
        self.y = torch.empty((T, O), dtype=torch.bfloat16, device=device)
        self.dX = torch.empty((T, I), dtype=torch.bfloat16, device=device)
        self.dW = torch.zeros((O, I), dtype=f32, device=device)

    def _check(self, t: torch.Tensor, shape, what: str):
        if tuple(t.shape) != shape:
            raise Fgfp8Error(f"{what} has shape {tuple(t.shape)}, expected {shape}")

    # casts -----------------------------------------------------------------------------
    def cast_input(self, x: torch.Tensor) -> None:
        """x -> xq/sx (groups along d_in) and xTq/sxT (groups along the tokens), one read."""
        self._check(x, (self.T, self.I), "x")
        if self.recipe == "fp32":
            cast_per_token_dual(x, self.xq, self.sx, self.xTq, self.sxT)
        elif self.recipe == "ue8m0":
            cast_per_token_dual(x, self.xq, self.sx, self.xTq, self.sxT, SF_UE8M0)
        else:
            cast_per_token_dual(x, self.xq, self.sx, self.xTq, self.sxT, SF_PACKED_UE8M0, 32)

    def cast_weight(self, W: torch.Tensor) -> None:
        """W -> Wq/sW and its transpose WqT/sWT (128 x 128 blocks; 1 x 32 groups in the
        group-32 recipe)."""
        self._check(W, (self.O, self.I), "W")
        if self.recipe == "fp32":
            cast_per_block(W, self.Wq, self.sW, self.WqT, self.sWT, SF_FP32)
        elif self.recipe == "ue8m0":
            cast_per_block(W, self.Wq, self.sW, self.WqT, self.sWT, SF_UE8M0)
        else:
            cast_per_token_dual(W, self.Wq, self.sW, self.WqT, self.sWT, SF_PACKED_UE8M0, 32)

    def cast_grad_output(self, dY: torch.Tensor) -> None:
        """dY -> dYq/sdY (groups along d_out) and dYTq/sdYT (groups along the tokens)."""
        self._check(dY, (self.T, self.O), "dY")
        if self.recipe == "fp32":
            cast_per_token_dual(dY, self.dYq, self.sdY, self.dYTq, self.sdYT)
        elif self.recipe == "ue8m0":
            cast_per_token_dual(dY, self.dYq, self.sdY, self.dYTq, self.sdYT, SF_UE8M0)
        else:
            cast_per_token_dual(dY, self.dYq, self.sdY, self.dYTq, self.sdYT, SF_PACKED_UE8M0, 32)

    # GEMMs -----------------------------------------------------------------------------
    def forward(self) -> torch.Tensor:
        """y = x W^T from the cast operands."""
        if self.recipe == "fp32":
            gemm_fp8_nt_bf16(self.xq, self.sx, self.Wq, self.sW, self.y)
        elif self.recipe == "ue8m0":
            gemm_fp8_nt_bf16_ue8m0(self.xq, self.sx, self.Wq, self.sW, self.y, SF_UE8M0)
        else:
            gemm_fp8_nt_bf16_ue8m0_g32(self.xq, self.sx, self.Wq, self.sW, self.y)
        return self.y

    def backward_data(self) -> torch.Tensor:
        """dX = dY W, against the FP8 transpose of W."""
        if self.recipe == "fp32":
            gemm_fp8_nt_bf16(self.dYq, self.sdY, self.WqT, self.sWT, self.dX)
        elif self.recipe == "ue8m0":
            gemm_fp8_nt_bf16_ue8m0(self.dYq, self.sdY, self.WqT, self.sWT, self.dX, SF_UE8M0)
        else:
            gemm_fp8_nt_bf16_ue8m0_g32(self.dYq, self.sdY, self.WqT, self.sWT, self.dX)
        return self.dX

    def backward_weight(self) -> torch.Tensor:
        """dW += dY^T x in fp32."""
        if self.recipe == "fp32":
            wgrad_gemm_fp8_nt_fp32(self.dYTq, self.sdYT, self.xTq, self.sxT, self.dW)
        elif self.recipe == "ue8m0":
            wgrad_gemm_fp8_nt_fp32_ue8m0(self.dYTq, self.sdYT, self.xTq, self.sxT, self.dW, SF_UE8M0)
        else:
            wgrad_gemm_fp8_nt_fp32_ue8m0_g32(self.dYTq, self.sdYT, self.xTq, self.sxT, self.dW)
        return self.dW

    # the whole step --------------------------------------------------------------------
    def ops(self, x: torch.Tensor, W: torch.Tensor, dY: torch.Tensor):
        """The step as (name, launch) pairs in order: cast x, cast W, forward, cast dY,
        dgrad, wgrad."""
        return [
            ("cast_x", lambda: self.cast_input(x)),
            ("cast_W", lambda: self.cast_weight(W)),
            ("gemm_fwd", self.forward),
            ("cast_dY", lambda: self.cast_grad_output(dY)),
            ("gemm_dgrad", self.backward_data),
            ("gemm_wgrad", self.backward_weight),
        ]

    def step(self, x: torch.Tensor, W: torch.Tensor, dY: torch.Tensor):
        """Run the whole step; returns (y, dX, dW)."""
        for _, launch in self.ops(x, W, dY):
            launch()
        return self.y, self.dX, self.dW
