"""Host-side checks of fine_grained_block_token_amd.linear.Fp8Linear: the recipe and
shape validation that runs before any launch (no GPU needed)."""
import pytest
import torch

from fine_grained_block_token_amd import Fgfp8Error
from fine_grained_block_token_amd.linear import RECIPES, Fp8Linear


def test_recipes():
    assert RECIPES == ("fp32", "ue8m0", "ue8m0_g32")
    with pytest.raises(Fgfp8Error):
        Fp8Linear(128, 128, 128, "bf16", device="cpu")


@pytest.mark.parametrize("shape", [(100, 128, 128), (128, 130, 128), (128, 128, 0), (0, 128, 128)])
def test_shapes_must_be_whole_k_blocks(shape):
    # tokens, d_in and d_out are each a GEMM's K in one of the three products
    with pytest.raises(Fgfp8Error):
        Fp8Linear(*shape, device="cpu")


@pytest.mark.parametrize("recipe", ["fp32", "ue8m0", "ue8m0_g32"])
def test_buffers_and_input_shapes(recipe):
    L = Fp8Linear(256, 384, 128, recipe, device="cpu")
    assert L.xq.shape == (256, 384) and L.xTq.shape == (384, 256)
    assert L.Wq.shape == (128, 384) and L.WqT.shape == (384, 128)
    assert L.dYq.shape == (256, 128) and L.dYTq.shape == (128, 256)
    assert L.y.shape == (256, 128) and L.dX.shape == (256, 384) and L.dW.shape == (128, 384)
    assert L.dW.dtype == torch.float32 and not L.dW.any()
    # MN-major LHS scales (stride(0) == 1), one per row and 128-wide K block
    assert L.sx.shape == (256, 3) and L.sx.stride(0) == 1
    assert L.sdYT.shape == (128, 2) and L.sdYT.stride(0) == 1
    if recipe == "ue8m0_g32":
        assert L.sW.shape == (128, 3) and L.sW.dtype == torch.int32
    else:
        assert L.sW.shape == (1, 3) and L.sWT.shape == (3, 1) and L.sW.dtype == torch.float32
    # a wrong input shape is refused before anything is launched
    with pytest.raises(Fgfp8Error):
        L.cast_input(torch.zeros(256, 128, dtype=torch.bfloat16))
    with pytest.raises(Fgfp8Error):
        L.cast_weight(torch.zeros(384, 128, dtype=torch.bfloat16))
    with pytest.raises(Fgfp8Error):
        L.cast_grad_output(torch.zeros(128, 256, dtype=torch.bfloat16))
