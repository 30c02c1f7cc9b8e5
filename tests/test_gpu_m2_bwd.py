"""Mamba-2 backward on the GPU (through the C ABI) against the fp64 oracle's
reverse-mode gradients (pinned to finite differences and to the broadcast
Mamba-1 gradients on the CPU).

Tolerance: the kernels compute in fp32 from the same (bf16- or fp32-valued)
inputs the oracle reads exactly.  A gradient element is a sum of up to
batch x L x headdim (dA, dD, dt_bias), heads x headdim (dB, dC), headdim x N
(ddt) or N (dx) products carried through an adjoint recursion whose length
is bounded by the decay; with unit roundoff 2^-24 and at most ~1e5
accumulated roundings the error stays below ~1e-3 of the typical size (rms)
of that gradient where its terms cancel, and below 1e-4 relative where
they do not: |gpu - ref| <= 1e-3 rms(ref) + 1e-4 |ref| per element.  The
chunked matrix form (the default for bf16 inputs and N >= 32) multiplies
fp32 operands as bf16 hi + lo pairs, whose products carry a relative error
near 2^-16 (1.5e-5), inside the same bound."""
import numpy as np
import pytest
import torch

import oracle
import selective_state_space_25_amd as ss
import synth
from parity import check_close, host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RMS_TOL, REL_TOL = 1e-3, 1e-4
GRADS = ("dx", "ddt", "dA", "dB", "dC", "dD", "dz", "ddt_bias", "dh0")


def _check(got, ref, names=GRADS):
    for k in names:
        if k not in got:
            continue
        g = host(got[k]).double().numpy()
        r = np.asarray(ref[k])
        scale = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
        check_close(g, r, (RMS_TOL * scale + 1e-30, REL_TOL), k)


def _case(batch, L, H, G, N, dtype, seed=0, dout_dtype=torch.float32, h0=False, **kw):
    m = synth.m2_inputs(batch, L, H, 64, G, N, dtype, seed=seed, device=DEV, **kw)
    dout = synth.m2_dout(batch, L, H, 64, dout_dtype, seed=seed, device=DEV)
    st = synth.m2_state(batch, H, 64, N, seed=seed, device=DEV) if h0 else None
    return m, dout, st


def _run(m, dout, softplus=True, h0=None):
    g = ss.mamba2_bwd(m["x"], m["dt"], m["A"], m["B"], m["C"], m.get("D"), m.get("z"), m.get("dt_bias"), dout,
                      softplus=softplus, h0=h0)
    torch.cuda.synchronize()
    r = oracle.m2_bwd(host(m["x"]), host(m["dt"]), host(m["A"]), host(m["B"]), host(m["C"]), host(m.get("D")),
                      host(m.get("z")), host(m.get("dt_bias")), host(dout), softplus=softplus,
                      h0=None if h0 is None else host(h0))
    return g, r


@pytest.mark.parametrize("L", [1, 7, 8, 9, 31, 32, 33, 64, 100, 301])
def test_lengths(gpu, L):
    m, dout, _ = _case(1, L, 4, 2, 32, torch.bfloat16, seed=L)
    _check(*_run(m, dout))


@pytest.mark.parametrize("N", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_state_sizes_and_dtypes(gpu, N, dtype):
    m, dout, _ = _case(2, 77, 4, 1, N, dtype, seed=N)
    _check(*_run(m, dout))


def test_groups_share_b_and_c(gpu):
    """dB and dC sum over the heads of each group only."""
    m, dout, _ = _case(2, 50, 8, 4, 32, torch.bfloat16, seed=3)
    _check(*_run(m, dout))


@pytest.mark.parametrize("softplus", [True, False])
def test_h0_and_softplus(gpu, softplus):
    m, dout, h0 = _case(1, 45, 2, 1, 64, torch.float32, seed=5 + int(softplus), h0=True)
    if not softplus:
        # Delta = dt itself then: keep it positive (the bias, drawn for the
        # softplus, is negative and would make the state grow without bound)
        m["dt"] = (m["dt"].abs() * 0.1).contiguous()
        m["dt_bias"] = None
    _check(*_run(m, dout, softplus=softplus, h0=h0))


def test_without_gate_skip_bias(gpu):
    m, dout, _ = _case(1, 40, 2, 1, 16, torch.bfloat16, seed=9, gate=False, skip=False, bias=False)
    g, r = _run(m, dout)
    assert "dz" not in g and "dD" not in g and "ddt_bias" not in g
    _check(g, r)


def test_bf16_dout(gpu):
    m, dout, _ = _case(1, 33, 2, 1, 32, torch.bfloat16, seed=11, dout_dtype=torch.bfloat16)
    _check(*_run(m, dout))


def test_reproducible_bitwise(gpu):
    m, dout, _ = _case(1, 200, 4, 1, 128, torch.bfloat16, seed=13)
    a = ss.mamba2_bwd(m["x"], m["dt"], m["A"], m["B"], m["C"], m["D"], m["z"], m["dt_bias"], dout)
    b = ss.mamba2_bwd(m["x"], m["dt"], m["A"], m["B"], m["C"], m["D"], m["z"], m["dt_bias"], dout)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_unaligned_tensors(gpu):
    """An x that is not 16-byte aligned takes the recurrent form: same results."""
    m, dout, _ = _case(1, 70, 2, 1, 64, torch.bfloat16, seed=31)
    buf = torch.empty(m["x"].numel() + 1, dtype=m["x"].dtype, device=DEV)
    xs = buf[1:].view(m["x"].shape)
    xs.copy_(m["x"])
    m["x"] = xs
    _check(*_run(m, dout))


def test_full_size_sampled(gpu):
    """The Mamba-2 multi-head workload (batch 8, L 4096, 32 heads x 64, N 128,
    one group): per-(batch, head) gradients of two heads in two batch
    elements, and dB/dC of a run whose dout is zero outside those heads (the
    other heads' adjoints then vanish), against the oracle on those heads."""
    w = synth.WORKLOADS["mamba2_mh"]
    m = synth.workload_inputs(w, seed=0, device=DEV)
    dout = synth.m2_dout(w.batch, w.seqlen, w.nheads, w.headdim, torch.float32, seed=0, device=DEV)
    heads = [3, 30]
    mask = torch.zeros(w.nheads, device=DEV)
    mask[heads] = 1.0
    dout = (dout * mask[None, None, :, None]).contiguous()
    g = ss.mamba2_bwd(m["x"], m["dt"], m["A"], m["B"], m["C"], m["D"], m["z"], m["dt_bias"], dout)
    torch.cuda.synchronize()
    for b in (0, 7):
        sub = {k: host(v[b:b + 1, :, heads]) if k in ("x", "dt", "z") else v for k, v in m.items()}
        r = oracle.m2_bwd(sub["x"], sub["dt"], host(m["A"])[heads], host(m["B"][b:b + 1]), host(m["C"][b:b + 1]),
                          host(m["D"])[heads], sub["z"], host(m["dt_bias"])[heads], host(dout[b:b + 1, :, heads]))
        got = {"dx": g["dx"][b:b + 1, :, heads], "ddt": g["ddt"][b:b + 1, :, heads], "dz": g["dz"][b:b + 1, :, heads],
               "dB": g["dB"][b:b + 1], "dC": g["dC"][b:b + 1]}
        _check(got, r, names=("dx", "ddt", "dz", "dB", "dC"))


def test_caller_workspace(gpu):
    """A caller-provided workspace gives the same gradients bit for bit; one
    byte too small is refused."""
    m, dout, _ = _case(1, 100, 4, 2, 64, torch.bfloat16, seed=17)
    args = (m["x"], m["dt"], m["A"], m["B"], m["C"], m["D"], m["z"], m["dt_bias"], dout)
    n = ss.mamba2_bwd_workspace_bytes(1, 100, 4, 64, 2, 64, ss.BF16, ss.F32)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    a = ss.mamba2_bwd(*args)
    b = ss.mamba2_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    with pytest.raises(ss.SelscanError):
        ss.mamba2_bwd(*args, workspace=ws[:n - 1])


# ---- the recurrent form (SELSCAN_M2_BWD_SSD=0), which the tests above reach
# only for fp32 inputs and N = 16 --------------------------------------------

@pytest.mark.parametrize("L", [1, 7, 31, 32, 33, 100, 301])
def test_recurrent_form_lengths(gpu, monkeypatch, L):
    monkeypatch.setenv("SELSCAN_M2_BWD_SSD", "0")
    m, dout, _ = _case(1, L, 4, 2, 32, torch.bfloat16, seed=100 + L)
    _check(*_run(m, dout))


@pytest.mark.parametrize("N", [32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_recurrent_form_state_sizes(gpu, monkeypatch, N, dtype):
    monkeypatch.setenv("SELSCAN_M2_BWD_SSD", "0")
    m, dout, _ = _case(2, 77, 4, 1, N, dtype, seed=N + 1)
    _check(*_run(m, dout))


@pytest.mark.parametrize("softplus", [True, False])
def test_recurrent_form_h0_softplus(gpu, monkeypatch, softplus):
    monkeypatch.setenv("SELSCAN_M2_BWD_SSD", "0")
    m, dout, h0 = _case(1, 70, 2, 1, 64, torch.float32, seed=7 + int(softplus), h0=True)
    if not softplus:
        m["dt"] = (m["dt"].abs() * 0.1).contiguous()
        m["dt_bias"] = None
    _check(*_run(m, dout, softplus=softplus, h0=h0))


def test_recurrent_form_groups_no_gate(gpu, monkeypatch):
    monkeypatch.setenv("SELSCAN_M2_BWD_SSD", "0")
    m, dout, _ = _case(2, 50, 8, 4, 32, torch.bfloat16, seed=21)
    _check(*_run(m, dout))
    m, dout, _ = _case(1, 40, 2, 1, 64, torch.bfloat16, seed=22, gate=False, skip=False, bias=False)
    _check(*_run(m, dout))
