"""Pins of the fp64 oracle to things other than itself.

Each test fixes the oracle against a closed form, a library routine, a brute
force written along a different route, or an invariant that the mathematics of
the selective scan guarantees.  Between them a dropped term, a wrong sign, a
wrong index or a transposed operand anywhere in the oracle fails at least one:

  term / mistake                      caught by
  sign of exp(Delta A)                geometric series, brute force, LTI conv.
  softplus on Delta / the bias index  prefix-sum (A = 0) against numpy logaddexp
  Delta*B*u input term                prefix sum, brute force
  sum over n in the read-out          brute force, LTI convolution, one-hot C
  D skip term / gate placement        C = 0 case, z = 0 case
  [B, N, L] layout of B and C         brute force with asymmetric B, C
  [D, N] layout of A                  brute force with asymmetric A
  [B, D, N] layout of last_state      one-hot C
  initial state h0                    split = whole (Mamba-1 and Mamba-2)
  [B, H, P, N] layout of Mamba-2 h0   x = 0 decay closed form, one-hot C
  Mamba-2 group/head mapping          Mamba-2 = broadcast Mamba-1, brute force

Sources of the definitions: the "Understanding Mamba and Selective State Space
Models (SSMs)" blog, sections 2.1 and 2.2 (recurrence, zero initial state,
softplus on Delta, read-out), and the Mamba README on the gittoolsai tool page
(Selective SSM, Mamba-2, Initialization).
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle

RTOL = 1e-12


def _rand_m1(rng, nb=2, nd=3, nn=4, nl=17, a_kind="random"):
    u = rng.standard_normal((nb, nd, nl))
    delta = rng.standard_normal((nb, nd, nl))
    if a_kind == "random":
        A = -rng.uniform(0.1, 3.0, size=(nd, nn))
    else:
        A = -np.tile(np.arange(1, nn + 1, dtype=float), (nd, 1))
    B = rng.standard_normal((nb, nn, nl))
    C = rng.standard_normal((nb, nn, nl))
    D = rng.standard_normal(nd)
    z = rng.standard_normal((nb, nd, nl))
    bias = np.log(np.expm1(rng.uniform(1e-3, 1e-1, size=nd)))
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, delta_bias=bias)


def _silu(z):
    return z * expit(z)


def _close(a, b, rtol=RTOL):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    np.testing.assert_allclose(a, b, rtol=0, atol=rtol * scale)


# ---------------------------------------------------------------- P1 prefix sum
@pytest.mark.parametrize("softplus", [True, False])
def test_a_zero_is_prefix_sum(softplus):
    """A = 0 gives exp(Delta A) = 1, so h_t = cumsum_s(Delta_s B_s u_s)."""
    rng = np.random.default_rng(1)
    x = _rand_m1(rng)
    x["A"] = np.zeros_like(x["A"])
    y, last = oracle.m1(**x, softplus=softplus)
    pre = x["delta"] + x["delta_bias"][None, :, None]
    dt = np.logaddexp(0.0, pre) if softplus else pre          # library softplus
    inc = dt[:, :, None, :] * x["B"][:, None, :, :] * x["u"][:, :, None, :]  # [b,d,n,t]
    h = np.cumsum(inc, axis=-1)
    yy = np.einsum("bnt,bdnt->bdt", x["C"], h) + x["D"][None, :, None] * x["u"]
    yy = yy * _silu(x["z"])
    _close(y, yy)
    _close(last, h[..., -1])


def test_softplus_extremes_through_prefix_sum():
    """Large positive and negative Delta pre-activations: softplus(50) ~ 50,
    softplus(-50) ~ e^-50, checked through the A = 0 prefix sum."""
    nb, nd, nn, nl = 1, 2, 1, 6
    delta = np.array([[[50.0, -50.0, 0.0, 30.0, -30.0, 1e-3]] * nd])
    u = np.ones((nb, nd, nl))
    x = dict(u=u, delta=delta, A=np.zeros((nd, nn)), B=np.ones((nb, nn, nl)),
             C=np.ones((nb, nn, nl)))
    y, last = oracle.m1(**x, softplus=True)
    ref = np.cumsum(np.logaddexp(0.0, delta[0, 0]))
    _close(y[0, 0], ref)
    assert y[0, 0, 2] - y[0, 0, 1] == pytest.approx(math.log(2.0), rel=1e-15)
    assert y[0, 0, 1] - y[0, 0, 0] == pytest.approx(math.exp(-50.0), rel=1e-6)


# ---------------------------------------------------------------- P2 freeze
def test_zero_delta_freezes_state():
    """Delta = 0 exactly (softplus off, delta = 0, no bias): h stays 0,
    last_state is exactly zero and y = D u silu(z)."""
    rng = np.random.default_rng(2)
    x = _rand_m1(rng)
    x["delta"] = np.zeros_like(x["delta"])
    x["delta_bias"] = None
    y, last = oracle.m1(**x, softplus=False)
    assert np.all(last == 0.0)
    # numpy's exp and the C library's may differ in the last bit: 4 ulp
    np.testing.assert_allclose(y, x["D"][None, :, None] * x["u"] * (x["z"] / (1 + np.exp(-x["z"]))),
                               rtol=1e-15, atol=0)


def test_zero_delta_window_keeps_state_bitwise():
    """A window where delta = -bias (softplus off, so Delta = 0 exactly)
    leaves the state bitwise unchanged across the window."""
    rng = np.random.default_rng(3)
    x = _rand_m1(rng, nl=30)
    t1, t2 = 10, 22
    x["delta"][:, :, t1:t2] = -x["delta_bias"][None, :, None]
    _, last_before = oracle.m1(**{k: (v[..., :t1] if k in ("u", "delta", "z", "B", "C") else v)
                                  for k, v in x.items()}, softplus=False)
    _, last_after = oracle.m1(**{k: (v[..., :t2] if k in ("u", "delta", "z", "B", "C") else v)
                                 for k, v in x.items()}, softplus=False)
    np.testing.assert_array_equal(last_before, last_after)


# ---------------------------------------------------------------- P3 brute force
def _brute_m1(x, softplus=True):
    """Unrolled sum of explicit decay products, pure Python floats:
    h_t[n] = sum_{s<=t} (prod_{r=s+1..t} exp(Delta_r A[d,n])) Delta_s B[b,n,s] u_s."""
    u, dl, A, B, C = x["u"], x["delta"], x["A"], x["B"], x["C"]
    D, z, bias = x.get("D"), x.get("z"), x.get("delta_bias")
    nb, nd, nl = u.shape
    nn = A.shape[1]
    y = np.zeros((nb, nd, nl))
    last = np.zeros((nb, nd, nn))
    for b in range(nb):
        for d in range(nd):
            dts = []
            for t in range(nl):
                v = float(dl[b, d, t]) + (float(bias[d]) if bias is not None else 0.0)
                dts.append(math.log(1.0 + math.exp(v)) if softplus else v)
            for t in range(nl):
                acc = 0.0
                for n in range(nn):
                    hs = 0.0
                    for s in range(t + 1):
                        prod = 1.0
                        for r in range(s + 1, t + 1):
                            prod *= math.exp(dts[r] * float(A[d, n]))
                        hs += prod * dts[s] * float(B[b, n, s]) * float(u[b, d, s])
                    acc += float(C[b, n, t]) * hs
                    if t == nl - 1:
                        last[b, d, n] = hs
                yv = acc + (float(D[d]) * float(u[b, d, t]) if D is not None else 0.0)
                if z is not None:
                    zz = float(z[b, d, t])
                    yv *= zz / (1.0 + math.exp(-zz))
                y[b, d, t] = yv
    return y, last


@pytest.mark.parametrize("softplus", [True, False])
def test_brute_force_tiny(softplus):
    rng = np.random.default_rng(4)
    x = _rand_m1(rng, nb=2, nd=3, nn=4, nl=12)
    if not softplus:  # keep Delta positive and moderate
        x["delta"] = np.abs(x["delta"]) * 0.3
        x["delta_bias"] = np.abs(x["delta_bias"]) * 0.01
    y, last = oracle.m1(**x, softplus=softplus)
    yb, lb = _brute_m1(x, softplus=softplus)
    _close(y, yb, 1e-11)
    _close(last, lb, 1e-11)


# ---------------------------------------------------------------- P4 LTI convolution
def test_time_invariant_case_is_causal_convolution():
    """Constant Delta, B, C over time: y = K * u + D u with
    K_k = sum_n C[n] exp(k Delta A[n]) Delta B[n]  (the classical SSM's
    convolution view)."""
    rng = np.random.default_rng(5)
    nb, nd, nn, nl = 1, 2, 5, 40
    A = -rng.uniform(0.05, 2.0, size=(nd, nn))
    Bv = rng.standard_normal(nn)
    Cv = rng.standard_normal(nn)
    dconst = rng.uniform(0.05, 0.5, size=nd)
    u = rng.standard_normal((nb, nd, nl))
    D = rng.standard_normal(nd)
    x = dict(u=u, delta=np.broadcast_to(dconst[None, :, None], (nb, nd, nl)).copy(), A=A,
             B=np.broadcast_to(Bv[None, :, None], (nb, nn, nl)).copy(),
             C=np.broadcast_to(Cv[None, :, None], (nb, nn, nl)).copy(), D=D)
    y, _ = oracle.m1(**x, softplus=False)
    k = np.arange(nl)
    for d in range(nd):
        K = (Cv[None, :] * np.exp(k[:, None] * dconst[d] * A[d][None, :]) * dconst[d] * Bv[None, :]).sum(1)
        ref = np.convolve(u[0, d], K)[:nl] + D[d] * u[0, d]
        _close(y[0, d], ref)


# ---------------------------------------------------------------- P5 geometric series
def test_geometric_series_closed_form():
    nl, a, dt = 50, 0.7, 0.3
    x = dict(u=np.ones((1, 1, nl)), delta=np.full((1, 1, nl), dt), A=np.array([[-a]]),
             B=np.ones((1, 1, nl)), C=np.ones((1, 1, nl)))
    y, last = oracle.m1(**x, softplus=False)
    q = math.exp(-a * dt)
    t = np.arange(nl)
    ref = dt * (1 - q ** (t + 1)) / (1 - q)
    _close(y[0, 0], ref)
    assert last[0, 0, 0] == pytest.approx(ref[-1], rel=1e-13)


# ---------------------------------------------------------------- P6 linearity
def test_linear_in_u():
    rng = np.random.default_rng(6)
    x = _rand_m1(rng)
    u1, u2 = x["u"], rng.standard_normal(x["u"].shape)
    al, be = 0.7, -1.9
    y1, l1 = oracle.m1(**x)
    y2, l2 = oracle.m1(**{**x, "u": u2})
    y3, l3 = oracle.m1(**{**x, "u": al * u1 + be * u2})
    _close(y3, al * y1 + be * y2)
    _close(l3, al * l1 + be * l2)


# ---------------------------------------------------------------- P7 causality
@pytest.mark.parametrize("name", ["u", "delta", "B", "C", "z"])
def test_causal(name):
    rng = np.random.default_rng(7)
    x = _rand_m1(rng, nl=25)
    y0, _ = oracle.m1(**x)
    t0 = 13
    x2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
    x2[name][..., t0] += 3.0
    y1, _ = oracle.m1(**x2)
    np.testing.assert_array_equal(y0[..., :t0], y1[..., :t0])
    assert not np.array_equal(y0[..., t0:], y1[..., t0:])


# ---------------------------------------------------------------- P8 zero prefix
def test_zero_input_prefix_shifts_output():
    rng = np.random.default_rng(8)
    x = _rand_m1(rng, nl=20)
    k = 7
    y0, l0 = oracle.m1(**x)
    pre = {n: rng.standard_normal(x[n].shape[:-1] + (k,)) for n in ("delta", "B", "C", "z")}
    pre["u"] = np.zeros(x["u"].shape[:-1] + (k,))
    x2 = {n: (np.concatenate([pre[n], v], axis=-1) if n in pre else v) for n, v in x.items()}
    y1, l1 = oracle.m1(**x2)
    np.testing.assert_array_equal(y1[..., k:], y0)
    np.testing.assert_array_equal(y1[..., :k], 0.0)
    np.testing.assert_array_equal(l1, l0)


# ---------------------------------------------------------------- P9 split = whole
def test_split_equals_whole_with_h0():
    rng = np.random.default_rng(9)
    x = _rand_m1(rng, nl=31)
    t1 = 12
    seq = ("u", "delta", "z", "B", "C")
    yw, lw = oracle.m1(**x)
    ya, la = oracle.m1(**{k: (v[..., :t1] if k in seq else v) for k, v in x.items()})
    yb, lb = oracle.m1(**{k: (v[..., t1:] if k in seq else v) for k, v in x.items()}, h0=la)
    _close(np.concatenate([ya, yb], axis=-1), yw, 1e-14)
    _close(lb, lw, 1e-14)


# ---------------------------------------------------------------- P10 one-hot C
def test_one_hot_c_reads_out_last_state():
    rng = np.random.default_rng(10)
    x = _rand_m1(rng, nb=2, nd=3, nn=5, nl=9)
    x["D"] = None
    x["z"] = None
    for k in range(5):
        C = x["C"].copy()
        C[:, :, -1] = 0.0
        C[:, k, -1] = 1.0
        y, last = oracle.m1(**{**x, "C": C})
        np.testing.assert_array_equal(y[:, :, -1], last[:, :, k])


# ---------------------------------------------------------------- P12 gate / skip
def test_c_zero_leaves_gated_skip():
    rng = np.random.default_rng(11)
    x = _rand_m1(rng)
    x["C"] = np.zeros_like(x["C"])
    y, _ = oracle.m1(**x)
    _close(y, x["D"][None, :, None] * x["u"] * _silu(x["z"]))


def test_z_zero_gives_zero_output():
    rng = np.random.default_rng(12)
    x = _rand_m1(rng)
    x["z"] = np.zeros_like(x["z"])
    y, _ = oracle.m1(**x)
    assert np.all(y == 0.0)


def test_softplus_of_zero_accumulates_ln2():
    nl = 9
    x = dict(u=np.ones((1, 1, nl)), delta=np.zeros((1, 1, nl)), A=np.zeros((1, 1)),
             B=np.ones((1, 1, nl)), C=np.ones((1, 1, nl)))
    y, _ = oracle.m1(**x, softplus=True)
    _close(y[0, 0], (np.arange(nl) + 1) * math.log(2.0))


def test_nan_propagates():
    rng = np.random.default_rng(13)
    x = _rand_m1(rng, nl=10)
    x["u"][0, 1, 4] = np.nan
    y, last = oracle.m1(**x)
    assert np.all(np.isnan(y[0, 1, 4:]))
    assert not np.any(np.isnan(y[0, 1, :4]))
    assert not np.any(np.isnan(y[0, 0]))
    assert np.all(np.isnan(last[0, 1]))


# ---------------------------------------------------------------- Mamba-2
def _rand_m2(rng, nb=2, nl=11, nh=4, npd=3, ng=2, nn=5):
    return dict(x=rng.standard_normal((nb, nl, nh, npd)), dt=rng.standard_normal((nb, nl, nh)),
                A=-rng.uniform(1.0, 16.0, size=nh), B=rng.standard_normal((nb, nl, ng, nn)),
                C=rng.standard_normal((nb, nl, ng, nn)), D=rng.standard_normal(nh),
                z=rng.standard_normal((nb, nl, nh, npd)),
                dt_bias=np.log(np.expm1(rng.uniform(1e-3, 1e-1, size=nh))))


def test_m2_equals_broadcast_m1():
    """Mamba-2 is Mamba-1 with A[d, n] = A_h, Delta shared by the P channels
    of a head, and the group's B/C broadcast to its heads."""
    rng = np.random.default_rng(14)
    m = _rand_m2(rng)
    nb, nl, nh, npd = m["x"].shape
    ng, nn = m["B"].shape[2:]
    y2, l2 = oracle.m2(**m)
    hpg = nh // ng
    for g in range(ng):
        heads = list(range(g * hpg, (g + 1) * hpg))
        u = np.concatenate([m["x"][:, :, h, :].transpose(0, 2, 1) for h in heads], axis=1)
        zz = np.concatenate([m["z"][:, :, h, :].transpose(0, 2, 1) for h in heads], axis=1)
        dl = np.concatenate([np.repeat(m["dt"][:, None, :, h], npd, axis=1) for h in heads], axis=1)
        A = np.concatenate([np.full((npd, nn), m["A"][h]) for h in heads], axis=0)
        Dv = np.concatenate([np.full(npd, m["D"][h]) for h in heads])
        bias = np.concatenate([np.full(npd, m["dt_bias"][h]) for h in heads])
        B1 = m["B"][:, :, g, :].transpose(0, 2, 1)
        C1 = m["C"][:, :, g, :].transpose(0, 2, 1)
        y1, l1 = oracle.m1(u=u, delta=dl, A=A, B=B1, C=C1, D=Dv, z=zz, delta_bias=bias)
        for i, h in enumerate(heads):
            _close(y2[:, :, h, :], y1[:, i * npd:(i + 1) * npd, :].transpose(0, 2, 1), 1e-13)
            _close(l2[:, h], l1[:, i * npd:(i + 1) * npd], 1e-13)


def test_m2_brute_force_tiny():
    rng = np.random.default_rng(15)
    m = _rand_m2(rng, nb=1, nl=8, nh=4, npd=2, ng=2, nn=3)
    y2, l2 = oracle.m2(**m)
    nb, nl, nh, npd = m["x"].shape
    ng, nn = m["B"].shape[2:]
    for b in range(nb):
        for h in range(nh):
            g = h // (nh // ng)
            dts = [math.log1p(math.exp(float(m["dt"][b, t, h] + m["dt_bias"][h]))) for t in range(nl)]
            for p in range(npd):
                for t in range(nl):
                    acc = 0.0
                    for n in range(nn):
                        hs = 0.0
                        for s in range(t + 1):
                            prod = math.exp(float(m["A"][h]) * sum(dts[s + 1:t + 1]))
                            hs += prod * dts[s] * m["B"][b, s, g, n] * m["x"][b, s, h, p]
                        acc += m["C"][b, t, g, n] * hs
                        if t == nl - 1:
                            assert l2[b, h, p, n] == pytest.approx(hs, rel=1e-11, abs=1e-13)
                    zz = m["z"][b, t, h, p]
                    ref = (acc + m["D"][h] * m["x"][b, t, h, p]) * zz / (1 + math.exp(-zz))
                    assert y2[b, t, h, p] == pytest.approx(ref, rel=1e-11, abs=1e-13)


def test_m2_one_hot_c_reads_out_last_state():
    rng = np.random.default_rng(16)
    m = _rand_m2(rng)
    m["D"] = None
    m["z"] = None
    nn = m["B"].shape[-1]
    for k in range(nn):
        C = m["C"].copy()
        C[:, -1] = 0.0
        C[:, -1, :, k] = 1.0
        y, last = oracle.m2(**{**m, "C": C})
        np.testing.assert_array_equal(y[:, -1], last[..., k])


# Mamba-2 from a carried state (blog section 2.2: the scan resumes from the
# state it was left in; README "Mamba-2": the state is [batch, heads, headdim,
# d_state]).  Two pins: splitting the sequence and resuming from the first
# part's last_state reproduces the whole; and with x = 0 the state only decays,
# h_t = exp(A_h sum_{s<=t} Delta_s) h0, so a one-hot C reads out h0 scaled by a
# closed-form factor -- which fixes h0's [B, H, P, N] layout on its own.
def test_m2_split_equals_whole_with_h0():
    rng = np.random.default_rng(17)
    m = _rand_m2(rng, nl=23)
    t1 = 9
    seq = ("x", "dt", "B", "C", "z")
    yw, lw = oracle.m2(**m)
    ya, la = oracle.m2(**{k: (v[:, :t1] if k in seq else v) for k, v in m.items()})
    yb, lb = oracle.m2(**{k: (v[:, t1:] if k in seq else v) for k, v in m.items()}, h0=la)
    _close(np.concatenate([ya, yb], axis=1), yw, 1e-14)
    _close(lb, lw, 1e-14)
    # a nonzero h0 must change the result (an ignored h0 would pass the above
    # only if la were zero, which it is not)
    assert np.max(np.abs(la)) > 1e-3


@pytest.mark.parametrize("softplus", [True, False])
def test_m2_h0_decays_in_closed_form(softplus):
    rng = np.random.default_rng(18)
    m = _rand_m2(rng, nb=2, nl=7, nh=4, npd=3, ng=2, nn=5)
    nb, nl, nh, npd = m["x"].shape
    nn = m["B"].shape[-1]
    m["x"] = np.zeros_like(m["x"])
    m["D"] = None
    m["z"] = None
    if not softplus:
        m["dt"] = np.abs(m["dt"]) * 0.3
        m["dt_bias"] = None
    h0 = rng.standard_normal((nb, nh, npd, nn))
    raw = m["dt"] + (m["dt_bias"][None, None, :] if m["dt_bias"] is not None else 0.0)
    dts = np.logaddexp(0.0, raw) if softplus else raw           # [nb, nl, nh]
    decay = np.exp(m["A"][None, None, :] * np.cumsum(dts, axis=1))   # [nb, nl, nh]
    for k in range(nn):
        C = np.zeros_like(m["C"])
        C[..., k] = 1.0
        y, last = oracle.m2(**{**m, "C": C}, softplus=softplus, h0=h0)
        ref = decay[:, :, :, None] * h0[:, None, :, :, k]       # [nb, nl, nh, npd]
        _close(y, ref, 1e-13)
    _close(last, decay[:, -1, :, None, None] * h0, 1e-13)


def test_bad_arguments_are_rejected():
    with pytest.raises(RuntimeError):
        m = _rand_m2(np.random.default_rng(0), nh=3, ng=2)
        oracle.m2(**m)


# ---------------------------------------------------------------- stored fixtures
@pytest.mark.parametrize("name", ["m1_small.json", "m2_small.json"])
def test_oracle_matches_stored_fixture(name):
    """Regression guard: the fixtures under tests/golden/ were written by
    tests/golden/make_golden.py from this oracle; any later change to the
    oracle's arithmetic shows up here."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    fx = json.load(open(path))
    ins = {k: np.array(v) for k, v in fx["inputs"].items()}
    fn = oracle.m1 if fx["kind"] == "m1" else oracle.m2
    y, last = fn(**ins, softplus=fx["softplus"])
    np.testing.assert_allclose(y, np.array(fx["y"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(last, np.array(fx["last_state"]), rtol=1e-14, atol=1e-15)


# ---- causal depthwise convolution (blog section 3.3; README causal-conv1d) --
#   term / mistake                 caught by
#   kernel orientation (k order)   numpy.convolve, shift kernel
#   causal offset / zero padding   shift kernel, numpy.convolve, causality
#   [dim, K] layout of w, bias     numpy.convolve with distinct rows
#   silu after the bias            numpy.convolve + scipy expit

@pytest.mark.parametrize("K", [1, 2, 4, 7])
@pytest.mark.parametrize("silu", [False, True])
def test_conv1d_matches_numpy_convolve(K, silu):
    rng = np.random.default_rng(100 + K)
    x = rng.standard_normal((2, 5, 23))
    w = rng.standard_normal((5, K))
    bias = rng.standard_normal(5)
    out = oracle.conv1d(x, w, bias, silu=silu)
    for b in range(2):
        for d in range(5):
            ref = np.convolve(x[b, d], w[d, ::-1])[:23] + bias[d]
            if silu:
                ref = _silu(ref)
            np.testing.assert_allclose(out[b, d], ref, rtol=RTOL, atol=1e-13)


def test_conv1d_identity_and_shift_kernels():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 3, 12))
    ident = np.zeros((3, 4))
    ident[:, 3] = 1.0
    assert np.array_equal(oracle.conv1d(x, ident, None, silu=False), x)
    shift = np.zeros((3, 4))
    shift[:, 0] = 1.0
    out = oracle.conv1d(x, shift, None, silu=False)
    assert np.array_equal(out[..., 3:], x[..., :-3])
    assert np.array_equal(out[..., :3], np.zeros((1, 3, 3)))


def test_conv1d_is_causal():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 4, 30))
    w = rng.standard_normal((4, 4))
    base = oracle.conv1d(x, w, None, silu=True)
    x2 = x.copy()
    x2[:, :, 17] += 3.0
    pert = oracle.conv1d(x2, w, None, silu=True)
    assert np.array_equal(base[..., :17], pert[..., :17])
    assert not np.array_equal(base[..., 17:21], pert[..., 17:21])
    assert np.array_equal(base[..., 21:], pert[..., 21:])


# ---- gradients of the Mamba-1 scan ----------------------------------------
# The hand-derived adjoint in oracle_m1_bwd_f64 is pinned to central finite
# differences of the (already pinned) forward oracle: a different route to
# every partial derivative.  A wrong time index of the adjoint's decay, a
# dropped path through h_{t-1}, a wrong softplus derivative or a missing sum
# over channels of dB/dC shows up as a mismatch.

def _loss(inp, dout, softplus):
    y, _ = oracle.m1(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                     inp["delta_bias"], softplus=softplus, h0=inp["h0"])
    return float(np.sum(y * dout))


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("gate_skip_bias", [True, False])
def test_backward_matches_finite_differences(softplus, gate_skip_bias):
    rng = np.random.default_rng(31 + int(softplus) + 2 * int(gate_skip_bias))
    nb, nd, nn, nl = 2, 2, 3, 7
    inp = {
        "u": rng.standard_normal((nb, nd, nl)),
        "delta": rng.standard_normal((nb, nd, nl)) * 0.5 + (0.0 if softplus else 1.0),
        "A": -rng.uniform(0.2, 2.0, (nd, nn)),
        "B": rng.standard_normal((nb, nn, nl)),
        "C": rng.standard_normal((nb, nn, nl)),
        "D": rng.standard_normal(nd) if gate_skip_bias else None,
        "z": rng.standard_normal((nb, nd, nl)) if gate_skip_bias else None,
        "delta_bias": rng.standard_normal(nd) * 0.3 if gate_skip_bias else None,
        "h0": rng.standard_normal((nb, nd, nn)) if gate_skip_bias else None,
    }
    dout = rng.standard_normal((nb, nd, nl))
    g = oracle.m1_bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                      inp["delta_bias"], dout, softplus=softplus, h0=inp["h0"])
    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
             "delta_bias": "ddelta_bias", "h0": "dh0"}
    eps = 1e-6
    for name, gname in names.items():
        if inp[name] is None:
            continue
        fd = np.zeros_like(inp[name])
        for idx in np.ndindex(*inp[name].shape):
            plus = {k: (None if v is None else v.copy()) for k, v in inp.items()}
            minus = {k: (None if v is None else v.copy()) for k, v in inp.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd[idx] = (_loss(plus, dout, softplus) - _loss(minus, dout, softplus)) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=2e-6, atol=2e-7, err_msg=gname)
    if not gate_skip_bias:
        assert np.all(g["dD"] == 0) and np.all(g["dz"] == 0) and np.all(g["ddelta_bias"] == 0)


# ---- gradients of the Mamba-2 scan ----------------------------------------
# oracle_m2_bwd_f64 is pinned the same way, to central finite differences of
# the (pinned) Mamba-2 forward oracle.  Two groups of two heads make every
# sum that Mamba-2's sharing implies visible: ddt over a head's channels,
# dA/dD/ddt_bias over batches, tokens and channels, dB/dC over the heads of
# a group and their channels (a sum over the wrong heads, or one head only,
# moves dB and dC away from the differences).

def _loss_m2(inp, dout, softplus):
    y, _ = oracle.m2(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["dt_bias"],
                     softplus=softplus, h0=inp["h0"])
    return float(np.sum(y * dout))


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("gate_skip_bias", [True, False])
def test_m2_backward_matches_finite_differences(softplus, gate_skip_bias):
    rng = np.random.default_rng(41 + int(softplus) + 2 * int(gate_skip_bias))
    nb, nl, nh, npd, ng, nn = 2, 6, 4, 2, 2, 3
    inp = {
        "x": rng.standard_normal((nb, nl, nh, npd)),
        "dt": rng.standard_normal((nb, nl, nh)) * 0.5 + (0.0 if softplus else 1.0),
        "A": -rng.uniform(0.2, 2.0, nh),
        "B": rng.standard_normal((nb, nl, ng, nn)),
        "C": rng.standard_normal((nb, nl, ng, nn)),
        "D": rng.standard_normal(nh) if gate_skip_bias else None,
        "z": rng.standard_normal((nb, nl, nh, npd)) if gate_skip_bias else None,
        "dt_bias": rng.standard_normal(nh) * 0.3 if gate_skip_bias else None,
        "h0": rng.standard_normal((nb, nh, npd, nn)) if gate_skip_bias else None,
    }
    dout = rng.standard_normal((nb, nl, nh, npd))
    g = oracle.m2_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["dt_bias"], dout,
                      softplus=softplus, h0=inp["h0"])
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz", "dt_bias": "ddt_bias",
             "h0": "dh0"}
    eps = 1e-6
    for name, gname in names.items():
        if inp[name] is None:
            continue
        fd = np.zeros_like(inp[name])
        for idx in np.ndindex(*inp[name].shape):
            plus = {k: (None if v is None else v.copy()) for k, v in inp.items()}
            minus = {k: (None if v is None else v.copy()) for k, v in inp.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd[idx] = (_loss_m2(plus, dout, softplus) - _loss_m2(minus, dout, softplus)) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=2e-6, atol=2e-7, err_msg=gname)
    if not gate_skip_bias:
        assert np.all(g["dD"] == 0) and np.all(g["dz"] == 0) and np.all(g["ddt_bias"] == 0)


def test_m2_backward_equals_broadcast_m1_backward():
    """One head per group and headdim channels that are Mamba-1 channels with
    A[d, n] = A[head] and delta[d, t] = dt[t, head]: the Mamba-2 gradients are
    the Mamba-1 ones, summed over a head's channels for dt, A, D and bias."""
    rng = np.random.default_rng(7)
    nb, nl, nh, npd, nn = 1, 5, 2, 3, 4
    x = rng.standard_normal((nb, nl, nh, npd))
    dt = rng.standard_normal((nb, nl, nh)) * 0.5
    A = -rng.uniform(0.2, 2.0, nh)
    B = rng.standard_normal((nb, nl, nh, nn))
    C = rng.standard_normal((nb, nl, nh, nn))
    D = rng.standard_normal(nh)
    z = rng.standard_normal((nb, nl, nh, npd))
    bias = rng.standard_normal(nh) * 0.3
    dout = rng.standard_normal((nb, nl, nh, npd))
    g2 = oracle.m2_bwd(x, dt, A, B, C, D, z, bias, dout)
    for hh in range(nh):
        u1 = np.transpose(x[:, :, hh, :], (0, 2, 1))                        # [nb, P, L]
        d1 = np.repeat(np.transpose(dt[:, :, hh:hh + 1], (0, 2, 1)), npd, axis=1)
        g1 = oracle.m1_bwd(u1, d1, np.full((npd, nn), A[hh]), np.transpose(B[:, :, hh, :], (0, 2, 1)),
                           np.transpose(C[:, :, hh, :], (0, 2, 1)), np.full(npd, D[hh]),
                           np.transpose(z[:, :, hh, :], (0, 2, 1)), np.full(npd, bias[hh]),
                           np.transpose(dout[:, :, hh, :], (0, 2, 1)))
        np.testing.assert_allclose(g2["dx"][:, :, hh, :], np.transpose(g1["du"], (0, 2, 1)), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g2["dz"][:, :, hh, :], np.transpose(g1["dz"], (0, 2, 1)), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g2["ddt"][:, :, hh], g1["ddelta"].sum(axis=1), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g2["dA"][hh], g1["dA"].sum(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g2["dD"][hh], g1["dD"].sum(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g2["ddt_bias"][hh], g1["ddelta_bias"].sum(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g2["dB"][:, :, hh, :], np.transpose(g1["dB"], (0, 2, 1)), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(g2["dC"][:, :, hh, :], np.transpose(g1["dC"], (0, 2, 1)), rtol=1e-12, atol=1e-13)
