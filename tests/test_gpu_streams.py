"""Two independent problems on two streams at once give the same bits as run one after
the other: the entry points keep no state between calls (apart from the documented
static scratch of gemm_fp8_nt_bf16_splitk_noalloc, which is not used here), so calls on
different streams with their own buffers and workspaces do not interact.  Both streams
have the default priority."""
import pytest
import torch

import fine_grained_block_token_amd as fg
import synth_inputs as si
from gpu_util import say

pytestmark = pytest.mark.gpu


def _problem(seed, T=512, I=2048, O=1024):
    u8, f32 = torch.uint8, torch.float32
    p = dict(
        x=si.randn((T, I), seed).cuda(), W=si.randn((O, I), seed + 1).cuda(),
        xq=torch.empty((T, I), dtype=u8, device="cuda"), sx=fg.mn_major_scales(T, I // 128),
        Wq=torch.empty((O, I), dtype=u8, device="cuda"), sW=torch.empty((O // 128, I // 128), dtype=f32, device="cuda"),
        xTq=torch.empty((I, T), dtype=u8, device="cuda"), sxT=fg.mn_major_scales(I, T // 128),
        y=torch.empty((T, O), dtype=torch.bfloat16, device="cuda"),
        dW=torch.zeros((I, I), dtype=f32, device="cuda"),
        y1=torch.empty((16, O), dtype=torch.bfloat16, device="cuda"),
    )
    p["ws"] = torch.empty((max(fg.gemm_fp8_nt_bf16_splitk_workspace(16, O, I), 4) // 4,), dtype=f32, device="cuda")
    return p


def _run(p):
    fg.cast_per_token(p["x"], p["xq"], p["sx"], 128, fg.SF_FP32)
    fg.cast_per_block(p["W"], p["Wq"], p["sW"], sf_fmt=fg.SF_FP32)
    fg.cast_per_token(p["x"].t(), p["xTq"], p["sxT"], 128, fg.SF_FP32)
    fg.gemm_fp8_nt_bf16(p["xq"], p["sx"], p["Wq"], p["sW"], p["y"])
    fg.wgrad_gemm_fp8_nt_fp32(p["xTq"], p["sxT"], p["xTq"], p["sxT"], p["dW"])
    fg.gemm_fp8_nt_bf16_splitk(p["xq"][:16], p["sx"][:16], p["Wq"], p["sW"], p["y1"], p["ws"])


OUT = ("xq", "sx", "Wq", "sW", "xTq", "sxT", "y", "dW", "y1")


def test_two_streams_match_serial(gpu):
    probs = [_problem(si.SEED_A), _problem(si.SEED_A + 100)]
    say("streams: serial reference")
    for p in probs:
        p["dW"].zero_()
        _run(p)
    torch.cuda.synchronize()
    ref = [{k: p[k].cpu().clone() for k in OUT} for p in probs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for r in range(3):
        say("streams: concurrent pass", r)
        for p in probs:
            for k in OUT:
                p[k].zero_()
        torch.cuda.synchronize()
        for s, p in zip(streams, probs):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                _run(p)
        torch.cuda.synchronize()
        for i, p in enumerate(probs):
            for k in OUT:
                assert torch.equal(p[k].cpu(), ref[i][k]), f"pass {r}, problem {i}: {k} differs"
