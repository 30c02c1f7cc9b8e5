"""Mamba-2 multi-head scan on the GPU (through the C ABI) against the oracle."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import selective_state_space_25_amd as ss
import synth
from parity import TOL_BF16, TOL_F32, check_close, host, oracle_m2_units, tol_for, tol_out_bf16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(inp, softplus=True, out_dtype=None):
    y, last = ss.mamba2_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp.get("D"), inp.get("z"),
                            inp.get("dt_bias"), softplus=softplus, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y, last


def _full_compare(inp, softplus=True, tol=None, out_dtype=None):
    y, last = _run(inp, softplus, out_dtype)
    yr, lr = oracle.m2(host(inp["x"]), host(inp["dt"]), host(inp["A"]), host(inp["B"]), host(inp["C"]),
                       host(inp.get("D")), host(inp.get("z")), host(inp.get("dt_bias")), softplus=softplus)
    tol = tol or tol_for(inp["x"].dtype)
    check_close(host(y).double().numpy(), yr, tol_out_bf16(tol) if y.dtype == torch.bfloat16 else tol, "y")
    check_close(host(last).double().numpy(), lr, tol, "last_state")
    return y, last


def _inputs(batch, L, H, P, G, N, dtype, seed=0, **kw):
    return synth.m2_inputs(batch, L, H, P, G, N, dtype, seed=seed, device=DEV, **kw)


@pytest.mark.parametrize("N", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_state_sizes(gpu, N, dtype):
    inp = _inputs(2, 150, 4, 64, 2, N, dtype, seed=N)
    _full_compare(inp)


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 513])
def test_lengths(gpu, L):
    inp = _inputs(1, L, 4, 64, 1, 128, torch.bfloat16, seed=L)
    _full_compare(inp)


@pytest.mark.parametrize("P", [1, 17, 64, 80, 130])
def test_head_dims(gpu, P):
    inp = _inputs(2, 90, 3, P, 3, 32, torch.bfloat16, seed=P)
    _full_compare(inp)


@pytest.mark.parametrize("chunks", [1, 2, 5, 33])
def test_chunk_carry_plans(gpu, monkeypatch, chunks):
    monkeypatch.setenv("SELSCAN_M2_CHUNKS", str(chunks))
    inp = _inputs(2, 700, 4, 64, 2, 64, torch.bfloat16, seed=chunks)
    _full_compare(inp)


@pytest.mark.parametrize("opt", ["no_gate", "no_skip", "no_bias", "bf16_out"])
def test_options(gpu, opt):
    kw = {"gate": opt != "no_gate", "skip": opt != "no_skip", "bias": opt != "no_bias"}
    inp = _inputs(1, 200, 4, 64, 1, 64, torch.bfloat16, seed=21, **kw)
    out_dtype = torch.bfloat16 if opt == "bf16_out" else None
    y, _ = _full_compare(inp, out_dtype=out_dtype)
    assert y.dtype == (out_dtype or torch.float32)


def test_golden_fixture(gpu):
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "m2_small.json")))
    ins = {k: torch.tensor(v, dtype=torch.float32, device=DEV) for k, v in fx["inputs"].items()}
    y, last = _run(ins, fx["softplus"])
    check_close(host(y).double().numpy(), np.array(fx["y"]), TOL_F32, "y")
    check_close(host(last).double().numpy(), np.array(fx["last_state"]), TOL_F32, "last_state")


def test_one_hot_c_pins_last_state_layout(gpu):
    inp = _inputs(1, 50, 4, 64, 2, 32, torch.float32, seed=9, gate=False, skip=False)
    for k in (0, 7, 31):
        C = inp["C"].clone()
        C[:, -1] = 0.0
        C[:, -1, :, k] = 1.0
        y, last = _run({**inp, "C": C})
        check_close(host(y[:, -1]).numpy(), host(last[..., k]).numpy(), (1e-6, 1e-6), "y vs last_state")


def test_deterministic(gpu):
    inp = _inputs(2, 500, 8, 64, 1, 128, torch.bfloat16, seed=8)
    y0, l0 = _run(inp)
    y1, l1 = _run(inp)
    assert torch.equal(y0, y1) and torch.equal(l0, l1)


@pytest.mark.parametrize("N,G", [(128, 2), (64, 4)])
def test_xcd_unit_order_is_a_permutation(gpu, monkeypatch, N, G):
    """The chunked matrix form's placement of (batch, head) units on the
    XCDs (16 units, a multiple of 8) only reorders the workgroups: y and the
    final state are bitwise those of the linear order, and match the oracle."""
    inp = _inputs(2, 200, 8, 64, G, N, torch.bfloat16, seed=N + G)
    y1, l1 = _full_compare(inp)
    monkeypatch.setenv("SELSCAN_M2_XCD_UNITS", "0")
    y0, l0 = _run(inp)
    assert torch.equal(y0, y1) and torch.equal(l0, l1)


def test_causality_bitwise(gpu, monkeypatch):
    monkeypatch.setenv("SELSCAN_M2_CHUNKS", "3")
    inp = _inputs(1, 300, 4, 64, 1, 64, torch.bfloat16, seed=3)
    y0, _ = _run(inp)
    t0 = 151
    x = inp["x"].clone()
    x[:, t0] += 1.0
    y1, _ = _run({**inp, "x": x})
    assert torch.equal(y0[:, :t0], y1[:, :t0])
    assert not torch.equal(y0[:, t0:], y1[:, t0:])


@pytest.mark.parametrize("N,G,L", [(64, 1, 200), (128, 2, 333), (128, 4, 64)])
def test_chunked_mfma_form_matches_recurrent_form(gpu, monkeypatch, N, G, L):
    """The chunked matrix form (bf16 inputs, headdim 64, N 64 or 128) and the
    recurrent form agree with each other and with the oracle."""
    inp = _inputs(2, L, 4, 64, G, N, torch.bfloat16, seed=N + G)
    y_ssd, l_ssd = _full_compare(inp)
    monkeypatch.setenv("SELSCAN_M2_SSD", "0")
    y_rec, l_rec = _full_compare(inp)
    check_close(host(y_ssd).double().numpy(), host(y_rec).double().numpy(), TOL_BF16, "y ssd vs recurrent")
    check_close(host(l_ssd).double().numpy(), host(l_rec).double().numpy(), TOL_BF16, "state ssd vs recurrent")


def test_full_size_workload_sampled(gpu):
    """Mamba-2 workload at full size: sampled (batch, head) units."""
    w = synth.WORKLOADS["mamba2_mh"]
    inp = synth.workload_inputs(w, device=DEV)
    y, last = _run(inp)
    units = [(0, 0), (w.batch - 1, w.nheads - 1), (3, 17), (5, 8)]
    yr, lr = oracle_m2_units(inp, units)
    for i, (b, h) in enumerate(units):
        check_close(host(y[b, :, h]).double().numpy(), yr[i], TOL_BF16, f"y unit {(b, h)}")
        check_close(host(last[b, h]).double().numpy(), lr[i], TOL_BF16, f"last unit {(b, h)}")


@pytest.mark.parametrize("form", ["split_roles", "shared_phases"])
@pytest.mark.parametrize("case", ["h0_n128_g2", "h0_n128_g2_bf16_out", "h0_single_token", "no_softplus",
                                  "group_per_head", "ragged_many_heads", "h0_n64_two_chunks"])
def test_chunked_mfma_form_edge_cases(gpu, monkeypatch, case, form):
    """The chunked matrix form (bf16 inputs, headdim 64, N 64 or 128), in
    both of its kernels (state and chunk waves with split roles, the default;
    all waves in every phase), on an initial state, a single token, softplus
    off, one group per head and a ragged length over several batches and
    heads, against the oracle."""
    monkeypatch.setenv("SELSCAN_M2_SSD_WS", "1" if form == "split_roles" else "0")
    N = 64 if case in ("group_per_head", "h0_single_token", "h0_n64_two_chunks") else 128
    L = {"h0_single_token": 1, "ragged_many_heads": 197, "h0_n64_two_chunks": 128}.get(case, 333)
    batch, H, G = (3, 6, 3) if case == "ragged_many_heads" else (2, 4, 4 if case == "group_per_head" else 2)
    inp = _inputs(batch, L, H, 64, G, N, torch.bfloat16, seed=len(case))
    softplus = case != "no_softplus"
    if not softplus:
        # Delta = dt + dt_bias must stay positive without softplus
        inp["dt"] = (inp["dt"].float().abs() * 0.05).to(torch.bfloat16)
        inp["dt_bias"] = inp["dt_bias"].abs() * 0.01
    h0 = None
    if case.startswith("h0"):
        g = torch.Generator(device=DEV).manual_seed(len(case))
        h0 = torch.randn((batch, H, 64, N), generator=g, device=DEV)
    out_dtype = torch.bfloat16 if case.endswith("bf16_out") else None
    y, last = ss.mamba2_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                            inp["dt_bias"], softplus=softplus, out_dtype=out_dtype, h0=h0)
    torch.cuda.synchronize()
    yr, lr = oracle.m2(host(inp["x"]), host(inp["dt"]), host(inp["A"]), host(inp["B"]), host(inp["C"]),
                       host(inp["D"]), host(inp["z"]), host(inp["dt_bias"]), softplus=softplus,
                       h0=None if h0 is None else host(h0))
    check_close(host(y).double().numpy(), yr, tol_out_bf16(TOL_BF16) if out_dtype else TOL_BF16, "y")
    check_close(host(last).double().numpy(), lr, TOL_BF16, "last_state")


@pytest.mark.parametrize("ssd", ["1", "0"])
def test_long_sequence_sampled(gpu, monkeypatch, ssd):
    """A million-token sequence with a ragged last chunk through the chunked
    matrix form (16,385 chunks walked by one workgroup per head) and through
    the recurrent form: sampled heads against the oracle over the whole
    length, and their final states."""
    monkeypatch.setenv("SELSCAN_M2_SSD", ssd)
    L = (1 << 20) + 37
    inp = _inputs(1, L, 4, 64, 1, 64, torch.bfloat16, seed=20)
    print(f"[m2 long] ssd={ssd} L={L}", flush=True)
    y, last = _run(inp)
    units = [(0, 0), (0, 3)]
    yr, lr = oracle_m2_units(inp, units)
    for i, (b, h) in enumerate(units):
        check_close(host(y[b, :, h]).double().numpy(), yr[i], TOL_BF16, f"y unit {(b, h)}")
        check_close(host(last[b, h]).double().numpy(), lr[i], TOL_BF16, f"last unit {(b, h)}")
    del inp, y, last, yr
    torch.cuda.empty_cache()
