"""Mamba-1 backward on the GPU (through the C ABI) against the fp64 oracle's
reverse-mode gradients (which are pinned to finite differences on the CPU).

Tolerance: the kernels compute in fp32 from the same (bf16- or fp32-valued)
inputs the oracle reads exactly, so the only error is fp32 arithmetic.  A
gradient element is a sum of up to batch x L (dA, dD, dbias), dim (dB, dC)
or N (du, ddelta) products carried through an adjoint recursion whose
effective length is bounded by the decay; with unit roundoff 2^-24 ~ 6e-8
and at most ~1e4 accumulated roundings the error stays below ~1e-3 of the
typical size (rms) of that gradient even where its terms cancel, and below
1e-4 relative where they do not.  Hence |gpu - ref| <= 1e-3 rms(ref) +
1e-4 |ref| per element."""
import ctypes

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
GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0")


def _check_grads(got, ref, names=GRADS, rows=None, chans=None):
    for k in names:
        if k not in got:
            continue
        g = host(got[k]).double().numpy()
        r = np.asarray(ref[k])
        if rows is not None and k in ("du", "ddelta", "dz", "dh0"):
            g = g[:, chans]
        if chans is not None and k in ("dA", "dD", "ddelta_bias"):
            g = g[chans]
        scale = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
        check_close(g, r, (RMS_TOL * scale + 1e-30, REL_TOL), k)


def _oracle(inp, dout, softplus=True, h0=None):
    return oracle.m1_bwd(host(inp["u"]), host(inp["delta"]), host(inp["A"]), host(inp["B"]), host(inp["C"]),
                         host(inp.get("D")), host(inp.get("z")), host(inp.get("delta_bias")), host(dout),
                         softplus=softplus, h0=None if h0 is None else host(h0))


def _gpu(inp, dout, softplus=True, h0=None, want_dh0=False):
    g = ss.bwd(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp.get("D"), inp.get("z"),
               inp.get("delta_bias"), dout, softplus=softplus, h0=h0, want_dh0=want_dh0)
    torch.cuda.synchronize()
    return g


def _case(batch, dim, N, L, dtype, a_kind="s4d_jitter", seed=0, dout_dtype=None, **kw):
    inp = synth.m1_inputs(batch, dim, N, L, dtype, a_kind, seed=seed, device=DEV, **kw)
    dout = synth.m1_dout(batch, dim, L, dout_dtype or torch.float32, seed=seed, device=DEV)
    return inp, dout


@pytest.mark.parametrize("L", [1, 17, 32, 33, 200, 1000])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_lengths(gpu, L, dtype):
    inp, dout = _case(2, 70, 16, L, dtype, seed=L)
    _check_grads(_gpu(inp, dout), _oracle(inp, dout))


@pytest.mark.parametrize("chunk", [32, 48, 64, 96, 512])
def test_chunked_time_matches_oracle(gpu, monkeypatch, chunk):
    """Chunks of the sequence linked by the state and adjoint carries (48: an
    odd number of 16-token tiles per chunk)."""
    monkeypatch.setenv("SELSCAN_BWD_CHUNK", str(chunk))
    inp, dout = _case(2, 130, 16, 1000, torch.bfloat16, seed=chunk)
    _check_grads(_gpu(inp, dout), _oracle(inp, dout))


@pytest.mark.parametrize("lane", ["0", "1"])
@pytest.mark.parametrize("dtype,dout_dtype,a_kind,gate", [
    (torch.bfloat16, torch.float32, "s4d_jitter", True), (torch.bfloat16, torch.bfloat16, "random", True),
    (torch.float32, torch.float32, "s4d", False), (torch.float32, torch.bfloat16, "random", True)])
def test_summary_pass_forms(gpu, monkeypatch, lane, dtype, dout_dtype, a_kind, gate):
    """Rows on 16-byte boundaries take the one-channel-per-lane summary pass
    unless it is switched off; both forms match the oracle with several
    chunks, a last chunk of one 32-token tile plus 8 tokens, a partial
    64-channel block, structured and general A, every dtype pair."""
    monkeypatch.setenv("SELSCAN_BWD_LANE_SUMMARY", lane)
    monkeypatch.setenv("SELSCAN_BWD_CHUNK", "64")
    inp, dout = _case(2, 100, 16, 1000, dtype, a_kind=a_kind, seed=5, dout_dtype=dout_dtype, gate=gate)
    _check_grads(_gpu(inp, dout), _oracle(inp, dout))


@pytest.mark.parametrize("images", ["0", "1"])
@pytest.mark.parametrize("dout_dtype,a_kind,gate,chunk", [
    (torch.float32, "s4d_jitter", True, "64"), (torch.bfloat16, "random", True, "96"),
    (torch.float32, "random", False, "32"), (torch.float32, "s4d", True, "0")])
def test_chunk_pass_row_images(gpu, monkeypatch, images, dout_dtype, a_kind, gate, chunk):
    """bf16 inputs with L and the chunk multiples of 32 take the chunk pass
    that reads 32-token row images from LDS unless it is switched off; both
    match the oracle (a partial 64-channel block, several chunks, a shorter
    last chunk for chunk 96)."""
    monkeypatch.setenv("SELSCAN_BWD_CHUNK_IMAGES", images)
    if chunk != "0":
        monkeypatch.setenv("SELSCAN_BWD_CHUNK", chunk)
    inp, dout = _case(2, 100, 16, 1024, torch.bfloat16, a_kind=a_kind, seed=9, dout_dtype=dout_dtype, gate=gate)
    _check_grads(_gpu(inp, dout), _oracle(inp, dout))


@pytest.mark.parametrize("N", [1, 3, 8, 16])
@pytest.mark.parametrize("a_kind", ["s4d", "random"])
def test_state_sizes(gpu, monkeypatch, N, a_kind):
    monkeypatch.setenv("SELSCAN_BWD_CHUNK", "64")
    inp, dout = _case(2, 40, N, 300, torch.bfloat16, a_kind, seed=N)
    _check_grads(_gpu(inp, dout), _oracle(inp, dout))


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("gate,skip,bias", [(True, True, True), (False, False, False), (True, False, True),
                                            (False, True, False)])
def test_options(gpu, softplus, gate, skip, bias):
    inp, dout = _case(2, 66, 16, 150, torch.float32, seed=3, gate=gate, skip=skip, bias=bias)
    if not softplus:
        # Delta = delta + bias must stay positive without softplus
        inp["delta"] = inp["delta"].abs() * 0.05
        if bias:
            inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
    got = _gpu(inp, dout, softplus=softplus)
    assert ("dz" in got) == gate and ("dD" in got) == skip and ("ddelta_bias" in got) == bias
    _check_grads(got, _oracle(inp, dout, softplus=softplus))


def test_bf16_dout(gpu):
    inp, dout = _case(1, 64, 16, 257, torch.bfloat16, seed=8, dout_dtype=torch.bfloat16)
    _check_grads(_gpu(inp, dout), _oracle(inp, dout))


@pytest.mark.parametrize("chunk", [0, 64])
@pytest.mark.parametrize("L", [400, 384])   # 384: the chunk pass's row images too
def test_initial_state_and_its_gradient(gpu, monkeypatch, chunk, L):
    if chunk:
        monkeypatch.setenv("SELSCAN_BWD_CHUNK", str(chunk))
    inp, dout = _case(2, 70, 16, L, torch.bfloat16, seed=11)
    h0 = synth.m1_state(2, 70, 16, seed=11, device=DEV)
    got = _gpu(inp, dout, h0=h0)
    _check_grads(got, _oracle(inp, dout, h0=h0))
    # without h0 the gradient of the (zero) initial state is still defined
    got0 = _gpu(inp, dout, want_dh0=True)
    ref0 = _oracle(inp, dout)
    _check_grads(got0, ref0, names=("dh0", "du"))


def test_gradients_are_reproducible_bit_for_bit(gpu):
    inp, dout = _case(2, 200, 16, 3000, torch.bfloat16, seed=5)
    a = _gpu(inp, dout)
    b = _gpu(inp, dout)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_unaligned_gradient_outputs(gpu):
    """du, ddelta and dz 4 bytes off a 16-byte boundary (possible for callers
    of the C ABI, not through this binding) take the chunk pass that stores
    one value at a time; the gradients are bitwise those of aligned outputs."""
    inp, dout = _case(2, 100, 16, 1024, torch.bfloat16, seed=13)
    ref = _gpu(inp, dout)
    batch, dim, L = inp["u"].shape

    def shifted(shape):   # contiguous, data pointer 4 bytes past an allocation
        return torch.zeros(int(np.prod(shape)) + 1, dtype=torch.float32, device=DEV)[1:].view(shape)

    g = {k: shifted(tuple(v.shape)) if k in ("du", "ddelta", "dz") else torch.zeros_like(v) for k, v in ref.items()}
    assert g["du"].data_ptr() % 16 == 4
    s = ss.Shape(batch, dim, inp["A"].shape[1], L, ss._dtype_code(inp["u"]), ss._dtype_code(dout), None, 0)
    ptr = lambda t: None if t is None else t.data_ptr()
    gp = lambda k: g[k].data_ptr() if k in g else None
    ss._check(ss.lib().selscan_bwd(
        ctypes.byref(s), ptr(inp["u"]), ptr(inp["delta"]), ptr(inp["A"]), ptr(inp["B"]), ptr(inp["C"]),
        ptr(inp.get("D")), ptr(inp.get("z")), ptr(inp.get("delta_bias")), 1, None, ptr(dout),
        gp("du"), gp("ddelta"), gp("dA"), gp("dB"), gp("dC"), gp("dD"), gp("dz"), gp("ddelta_bias"), None,
        torch.cuda.current_stream(DEV).cuda_stream))
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(g[k], ref[k]), k


def test_gradient_matches_the_forward_by_directional_derivative(gpu):
    """<dout, d out/du . v> from the GPU forward (a central difference in
    fp32 along a random direction v) equals <du, v> from the GPU backward:
    the two entry points agree with each other as well as with the oracle."""
    inp, dout = _case(1, 64, 16, 256, torch.float32, seed=21)
    got = _gpu(inp, dout)
    g = torch.Generator(device=DEV).manual_seed(4)
    v = torch.randn(inp["u"].shape, generator=g, device=DEV)
    eps = 0.5

    def loss(u):
        y, _ = ss.fwd(u, inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["delta_bias"])
        return float((y.double() * dout.double()).sum())

    fd = (loss(inp["u"] + eps * v) - loss(inp["u"] - eps * v)) / (2 * eps)
    an = float((got["du"].double() * v.double()).sum())
    # the scan is linear in u given delta, so the difference quotient is exact
    # up to the forward's fp32 rounding of two large sums
    assert abs(fd - an) <= 1e-3 * max(1.0, abs(an)), (fd, an)


@pytest.mark.parametrize("name", ["mamba130m_l2k", "mamba2p8b_l8k", "long_1m"])
def test_full_size_sampled(gpu, name):
    """The workload's full shape, in the launch plan the benchmark times.
    Per-row gradients and the per-channel sums (dA, dD, dbias) of a sample
    of channels spread over the channel blocks are exact from the oracle
    run on those channels alone.  dB and dC sum over all channels: with
    dout zero outside the sample, the other channels' adjoints vanish, so the
    oracle on the sample gives them exactly too."""
    w = synth.WORKLOADS[name]
    inp = synth.workload_inputs(w, seed=1, device=DEV)
    dout = synth.m1_dout(w.batch, w.dim, w.seqlen, torch.float32, seed=1, device=DEV)
    chans = torch.arange(3, w.dim, 197).tolist()
    chans = sorted(set(chans + [0, w.dim - 1]))
    idx = torch.tensor(chans, device=DEV)
    sub = {k: (None if v is None else
               v.index_select(1, idx).contiguous() if k in ("u", "delta", "z") else
               v.index_select(0, idx).contiguous() if k in ("A", "D", "delta_bias") else v)
           for k, v in inp.items()}
    print(f"[bwd full size] {name} channels={len(chans)}", flush=True)
    ref = _oracle(sub, dout.index_select(1, idx))
    got = _gpu(inp, dout)
    # the sampled channels' rows, selected on the device (the 1M-token
    # gradients are 8.6 GB each)
    got = {k: (v.index_select(1, idx) if k in ("du", "ddelta", "dz") else v) for k, v in got.items()}
    _check_grads(got, ref, names=("du", "ddelta", "dz", "dA", "dD", "ddelta_bias"), chans=chans)
    del got
    masked = torch.zeros_like(dout)
    masked[:, idx] = dout[:, idx]
    got = _gpu(inp, masked)
    _check_grads(got, ref, names=("dB", "dC"))
    del got, masked, inp, dout
    torch.cuda.empty_cache()


def test_maximum_seqlen_sampled(gpu):
    """The longest sequence the backward accepts (2^22 tokens, 32-bit byte
    offsets from per-workgroup bases): per-row and per-channel gradients of
    sampled channels exact from the oracle on those channels, dB and dC
    from a run with dout zero outside the sample (as in the full-size
    test above)."""
    L = 1 << 22
    inp, dout = _case(1, 64, 16, L, torch.bfloat16, seed=22)
    chans = [0, 37, 63]
    idx = torch.tensor(chans, device=DEV)
    sub = {k: (None if v is None else
               v.index_select(1, idx).contiguous() if k in ("u", "delta", "z") else
               v.index_select(0, idx).contiguous() if k in ("A", "D", "delta_bias") else v)
           for k, v in inp.items()}
    print(f"[bwd max seqlen] B=1 D=64 L={L}", flush=True)
    ref = _oracle(sub, dout.index_select(1, idx))
    got = _gpu(inp, dout)
    got = {k: (v.index_select(1, idx) if k in ("du", "ddelta", "dz") else v) for k, v in got.items()}
    _check_grads(got, ref, names=("du", "ddelta", "dz", "dA", "dD", "ddelta_bias"), chans=chans)
    del got
    masked = torch.zeros_like(dout)
    masked[:, idx] = dout[:, idx]
    got = _gpu(inp, masked)
    _check_grads(got, ref, names=("dB", "dC"))
    del got, masked, inp, dout
    torch.cuda.empty_cache()
