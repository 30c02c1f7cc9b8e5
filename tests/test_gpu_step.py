"""Initial state (h0) and one-token decoding on the GPU, through the C ABI,
against the fp64 oracle (which takes h0 and is pinned by the split-equals-
whole property in the CPU pins)."""
import pytest
import torch

import oracle
import selective_state_space_25_amd as ss
import synth
from parity import TOL_BF16, TOL_F32, check_close, host, tol_for

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _h0(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(DEV)


def _m1_oracle(inp, h0=None, softplus=True):
    return oracle.m1(host(inp["u"]), host(inp["delta"]), host(inp["A"]), host(inp["B"]), host(inp["C"]),
                     host(inp.get("D")), host(inp.get("z")), host(inp.get("delta_bias")), softplus=softplus,
                     h0=None if h0 is None else host(h0))


def _m2_oracle(inp, h0=None):
    return oracle.m2(host(inp["x"]), host(inp["dt"]), host(inp["A"]), host(inp["B"]), host(inp["C"]),
                     host(inp.get("D")), host(inp.get("z")), host(inp.get("dt_bias")),
                     h0=None if h0 is None else host(h0))


@pytest.mark.parametrize("chunks", [1, 3, 8])
@pytest.mark.parametrize("general", [False, True])
def test_m1_fwd_h0_matches_oracle(gpu, monkeypatch, chunks, general):
    monkeypatch.setenv("SELSCAN_M1_CHUNKS", str(chunks))
    if general:
        monkeypatch.setenv("SELSCAN_FORCE_GENERAL", "1")
    inp = synth.m1_inputs(2, 130, 16, 700, torch.bfloat16, "s4d_jitter", seed=51, device=DEV)
    h0 = _h0((2, 130, 16), 5)
    y, last = ss.fwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                     inp["delta_bias"], h0=h0)
    torch.cuda.synchronize()
    yr, lr = _m1_oracle(inp, h0)
    check_close(host(y).double().numpy(), yr, TOL_BF16, "y")
    check_close(host(last).double().numpy(), lr, TOL_BF16, "last_state")


def test_m1_split_sequence_equals_whole(gpu):
    """Scanning a sequence in two calls, the second from the first's final
    state, reproduces the scan of the whole sequence (within tolerance of the
    oracle of the whole)."""
    inp = synth.m1_inputs(2, 96, 16, 900, torch.bfloat16, "s4d", seed=52, device=DEV)
    L1 = 413
    part = lambda t, sl: t[..., sl].contiguous() if t is not None and t.dim() == 3 else t
    a = {k: part(v, slice(0, L1)) for k, v in inp.items()}
    b = {k: part(v, slice(L1, None)) for k, v in inp.items()}
    _, last1 = ss.fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["delta_bias"])
    y2, last2 = ss.fwd(b["u"], b["delta"], b["A"], b["B"], b["C"], b["D"], b["z"], b["delta_bias"], h0=last1)
    torch.cuda.synchronize()
    yr, lr = _m1_oracle(inp)
    check_close(host(y2).double().numpy(), yr[..., L1:], TOL_BF16, "y of the second part")
    check_close(host(last2).double().numpy(), lr, TOL_BF16, "final state")


def _m1_steps(inp, state, T, softplus=True, with_gate=True):
    ys = []
    for t in range(T):
        sl = lambda v: v[..., t].contiguous()
        ys.append(ss.step(state, sl(inp["u"]), sl(inp["delta"]), inp["A"], sl(inp["B"]), sl(inp["C"]),
                          inp.get("D"), sl(inp["z"]) if with_gate else None, inp.get("delta_bias"),
                          softplus=softplus))
    torch.cuda.synchronize()
    return torch.stack(ys, dim=-1)


@pytest.mark.parametrize("N", [1, 3, 4, 8, 16])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_m1_step_matches_oracle(gpu, N, dtype):
    T = 9
    inp = synth.m1_inputs(3, 70, N, T, dtype, "random", seed=60 + N, device=DEV)
    h0 = _h0((3, 70, N), 6)
    state = h0.clone()
    y = _m1_steps(inp, state, T)
    yr, lr = _m1_oracle(inp, h0)
    tol = tol_for(dtype)
    check_close(host(y).double().numpy(), yr, tol, "y over the steps")
    check_close(host(state).double().numpy(), lr, tol, "state after the steps")


@pytest.mark.parametrize("softplus", [True, False])
def test_m1_step_options(gpu, softplus):
    T = 5
    inp = synth.m1_inputs(2, 64, 16, T, torch.float32, "s4d", seed=71, device=DEV, skip=False, bias=softplus)
    if not softplus:
        inp["delta"] = inp["delta"].abs() * 0.05   # positive Delta without softplus
    state = torch.zeros((2, 64, 16), dtype=torch.float32, device=DEV)
    y = _m1_steps(inp, state, T, softplus=softplus, with_gate=False)
    no_gate = dict(inp, z=None)
    yr, lr = _m1_oracle(no_gate, softplus=softplus)
    check_close(host(y).double().numpy(), yr, TOL_F32, "y")
    check_close(host(state).double().numpy(), lr, TOL_F32, "state")


def test_m1_steps_continue_a_scan(gpu):
    """A prompt scanned with fwd, then tokens decoded with step from its
    final state, equals the oracle of the whole sequence."""
    inp = synth.m1_inputs(2, 100, 16, 260, torch.bfloat16, "s4d_jitter", seed=73, device=DEV)
    Lp = 250
    pre = {k: (v[..., :Lp].contiguous() if v is not None and v.dim() == 3 else v) for k, v in inp.items()}
    _, state = ss.fwd(pre["u"], pre["delta"], pre["A"], pre["B"], pre["C"], pre["D"], pre["z"], pre["delta_bias"])
    tail = {k: (v[..., Lp:].contiguous() if v is not None and v.dim() == 3 else v) for k, v in inp.items()}
    y = _m1_steps(tail, state, 260 - Lp)
    yr, lr = _m1_oracle(inp)
    check_close(host(y).double().numpy(), yr[..., Lp:], TOL_BF16, "decoded y")
    check_close(host(state).double().numpy(), lr, TOL_BF16, "state")


@pytest.mark.parametrize("chunks", [1, 4])
def test_m2_fwd_h0_matches_oracle(gpu, monkeypatch, chunks):
    monkeypatch.setenv("SELSCAN_M2_CHUNKS", str(chunks))
    inp = synth.m2_inputs(2, 300, 4, 64, 2, 64, torch.bfloat16, seed=81, device=DEV)
    h0 = _h0((2, 4, 64, 64), 8)
    y, last = ss.mamba2_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                            inp["dt_bias"], h0=h0)
    torch.cuda.synchronize()
    yr, lr = _m2_oracle(inp, h0)
    check_close(host(y).double().numpy(), yr, TOL_BF16, "y")
    check_close(host(last).double().numpy(), lr, TOL_BF16, "last_state")


@pytest.mark.parametrize("N", [16, 32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_m2_step_matches_oracle(gpu, N, dtype):
    T = 6
    inp = synth.m2_inputs(2, T, 6, 20, 3, N, dtype, seed=90 + N, device=DEV)
    h0 = _h0((2, 6, 20, N), 9)
    state = h0.clone()
    ys = []
    for t in range(T):
        ys.append(ss.mamba2_step(state, inp["x"][:, t].contiguous(), inp["dt"][:, t].contiguous(), inp["A"],
                                 inp["B"][:, t].contiguous(), inp["C"][:, t].contiguous(), inp["D"],
                                 inp["z"][:, t].contiguous(), inp["dt_bias"]))
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1)
    yr, lr = _m2_oracle(inp, h0)
    tol = tol_for(dtype)
    check_close(host(y).double().numpy(), yr, tol, "y over the steps")
    check_close(host(state).double().numpy(), lr, tol, "state after the steps")


def test_step_does_not_touch_other_rows(gpu):
    """Rows past the end of a 256-thread block are not written."""
    T = 1
    inp = synth.m1_inputs(1, 5, 16, T, torch.float32, "s4d", seed=95, device=DEV)
    big = torch.full((1, 6, 16), 7.0, dtype=torch.float32, device=DEV)
    state = big[:, :5]
    assert state.is_contiguous()
    _m1_steps(inp, state, T)
    assert torch.equal(host(big[:, 5]), torch.full((1, 16), 7.0))


@pytest.mark.parametrize("N", [64, 128])
def test_m2_step_does_not_touch_other_rows(gpu, N):
    """Mamba-2 rows (eight states per thread here) past the last one of a
    partly filled block are not written: the state is followed by a guard."""
    inp = synth.m2_inputs(1, 1, 3, 5, 1, N, torch.float32, seed=97, device=DEV)
    rows = 3 * 5
    buf = torch.full(((rows + 3) * N,), 7.0, dtype=torch.float32, device=DEV)
    state = buf[:rows * N].view(1, 3, 5, N)
    state.zero_()
    sl = lambda k: inp[k][:, 0].contiguous()
    ss.mamba2_step(state, sl("x"), sl("dt"), inp["A"], sl("B"), sl("C"), inp["D"], sl("z"), inp["dt_bias"])
    torch.cuda.synchronize()
    assert torch.equal(host(buf[rows * N:]), torch.full((3 * N,), 7.0))
    assert not torch.equal(host(state), torch.zeros((1, 3, 5, N)))


@pytest.mark.parametrize("mamba2", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_step_with_unaligned_b_c(gpu, mamba2, dtype):
    """B and C starting one element past an aligned address take the
    element-wise loads of the step kernels and give the same result."""
    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    if mamba2:
        inp = synth.m2_inputs(2, 1, 4, 16, 2, 64, dtype, seed=95, device=DEV)
        sl = lambda k: inp[k][:, 0].contiguous()
        args = lambda B, C: (sl("x"), sl("dt"), inp["A"], B, C, inp["D"], sl("z"), inp["dt_bias"])
        run = lambda st, B, C: ss.mamba2_step(st, *args(B, C))
        h0 = _h0((2, 4, 16, 64), 11)
    else:
        inp = synth.m1_inputs(2, 48, 16, 1, dtype, "s4d_jitter", seed=96, device=DEV)
        sl = lambda k: inp[k][..., 0].contiguous()
        args = lambda B, C: (sl("u"), sl("delta"), inp["A"], B, C, inp["D"], sl("z"), inp["delta_bias"])
        run = lambda st, B, C: ss.step(st, *args(B, C))
        h0 = _h0((2, 48, 16), 12)
    B, C = sl("B"), sl("C")
    Bs, Cs = shifted(B), shifted(C)
    assert Bs.data_ptr() % 8 != 0 and Cs.data_ptr() % 8 != 0
    s_al, s_un = h0.clone(), h0.clone()
    y_al = run(s_al, B, C)
    y_un = run(s_un, Bs, Cs)
    torch.cuda.synchronize()
    assert torch.equal(y_al, y_un)
    assert torch.equal(s_al, s_un)


@pytest.mark.parametrize("mamba2", [False, True])
def test_bound_step_in_a_decoding_loop(gpu, mamba2):
    """bind_step / bind_mamba2_step marshal the arguments once; the loop
    refills the same token buffers in place and calls again.  The tokens
    decoded this way equal the oracle from the same initial state."""
    T = 7
    if mamba2:
        inp = synth.m2_inputs(2, T, 4, 24, 2, 64, torch.bfloat16, seed=97, device=DEV)
        h0 = _h0((2, 4, 24, 64), 11)
        cur = {k: inp[k][:, 0].clone() for k in ("x", "dt", "B", "C", "z")}
        state = h0.clone()
        call, y = ss.bind_mamba2_step(state, cur["x"], cur["dt"], inp["A"], cur["B"], cur["C"], inp["D"],
                                      cur["z"], inp["dt_bias"])
        ref_y, ref_last = _m2_oracle(inp, h0)
    else:
        inp = synth.m1_inputs(2, 90, 16, T, torch.bfloat16, "s4d_jitter", seed=98, device=DEV)
        h0 = _h0((2, 90, 16), 12)
        cur = {k: inp[k][..., 0].clone() for k in ("u", "delta", "B", "C", "z")}
        state = h0.clone()
        call, y = ss.bind_step(state, cur["u"], cur["delta"], inp["A"], cur["B"], cur["C"], inp["D"], cur["z"],
                               inp["delta_bias"])
        ref_y, ref_last = _m1_oracle(inp, h0)
    ys = []
    for t in range(T):
        for k, v in cur.items():
            v.copy_(inp[k][:, t] if mamba2 else inp[k][..., t])
        call()
        ys.append(y.clone())
    torch.cuda.synchronize()
    got = torch.stack(ys, dim=1 if mamba2 else -1)
    check_close(host(got).double().numpy(), ref_y, TOL_BF16, "y over the bound steps")
    check_close(host(state).double().numpy(), ref_last, TOL_BF16, "state after the bound steps")
