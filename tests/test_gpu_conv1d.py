"""Causal depthwise convolution on the GPU, through the C ABI, against the
fp64 oracle (pinned to numpy.convolve and special kernels)."""
import pytest
import torch

import oracle
import selective_state_space_25_amd as ss
from parity import TOL_BF16, TOL_F32, check_close, host, tol_out_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(batch, dim, L, K, dtype, seed, bias=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((batch, dim, L), generator=g, dtype=torch.float32).to(dtype).to(DEV)
    w = (torch.randn((dim, K), generator=g, dtype=torch.float32) * 0.5).to(DEV)
    b = torch.randn((dim,), generator=g, dtype=torch.float32).to(DEV) if bias else None
    return x, w, b


def _check(x, w, b, silu, out_dtype=None):
    out = ss.conv1d(x, w, b, silu=silu, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.conv1d(host(x), host(w), None if b is None else host(b), silu=silu)
    # the kernel computes in fp32 from exact inputs: fp32 tolerance, plus the
    # rounding of a bf16 output
    tol = tol_out_bf16(TOL_F32) if out.dtype == torch.bfloat16 else TOL_F32
    check_close(host(out).double().numpy(), ref, tol, "conv1d out")
    return out


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 8, 13])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_widths_and_dtypes(gpu, K, dtype):
    x, w, b = _inputs(2, 70, 96, K, dtype, seed=K)
    _check(x, w, b, silu=True)


@pytest.mark.parametrize("L", [1, 3, 7, 8, 9, 40, 64, 1001, 4104])
def test_lengths_and_ragged_rows(gpu, L):
    x, w, b = _inputs(2, 33, L, 4, torch.bfloat16, seed=L)
    _check(x, w, b, silu=True)


@pytest.mark.parametrize("silu,bias", [(False, False), (False, True), (True, False)])
def test_options(gpu, silu, bias):
    x, w, b = _inputs(3, 40, 128, 4, torch.float32, seed=3, bias=bias)
    _check(x, w, b, silu=silu)


def test_output_dtype_differs_from_input(gpu):
    x, w, b = _inputs(2, 64, 256, 4, torch.bfloat16, seed=11)
    out = _check(x, w, b, silu=True, out_dtype=torch.float32)
    assert out.dtype == torch.float32


def test_causal_bitwise(gpu):
    x, w, b = _inputs(1, 16, 200, 4, torch.bfloat16, seed=12)
    y0 = ss.conv1d(x, w, b)
    x2 = x.clone()
    x2[:, :, 100] += 1.0
    y1 = ss.conv1d(x2, w, b)
    torch.cuda.synchronize()
    assert torch.equal(y0[..., :100], y1[..., :100])
    assert torch.equal(y0[..., 104:], y1[..., 104:])


def test_conv_then_scan_matches_oracle_chain(gpu):
    """u = silu(conv(x)) feeding the scan: the GPU chain against the oracle
    chain run on the same bf16 u (the conv output is rounded to bf16, the
    scan's input type, on both sides)."""
    import synth
    inp = synth.m1_inputs(2, 96, 16, 300, torch.bfloat16, "s4d", seed=13, device=DEV)
    x, w, b = _inputs(2, 96, 300, 4, torch.bfloat16, seed=14)
    u = ss.conv1d(x, w, b, silu=True)
    y, last = ss.fwd(u, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"])
    torch.cuda.synchronize()
    u_ref = torch.tensor(oracle.conv1d(host(x), host(w), host(b), silu=True)).to(torch.bfloat16)
    # both sides' u agree to one bf16 rounding; feed the oracle the GPU's u
    check_close(host(u).double().numpy(), u_ref.double().numpy(), (2 ** -7, 2 ** -7), "u")
    yr, lr = oracle.m1(host(u), host(inp["delta"]), host(inp["A"]), host(inp["B"]), host(inp["C"]),
                       host(inp["D"]), host(inp["z"]), host(inp["delta_bias"]))
    check_close(host(y).double().numpy(), yr, TOL_BF16, "y")
    check_close(host(last).double().numpy(), lr, TOL_BF16, "last_state")
