"""Seeded synthetic inputs for the selective-scan workloads.

This module only draws random numbers with the distributions, shapes and
dtypes of the five workloads; it performs none of the scan's arithmetic.  The
same tensors (the same bytes) feed the HIP library and the fp64 oracle.

Every tensor gets its own generator stream, seeded from (seed, tensor id), so
adding or resizing one tensor never shifts another.  Large tensors are drawn on
the device they will live on (torch's counter-based generator on the GPU);
small parameter vectors are always drawn on the CPU so they are identical
whatever the device.

Distributions (the workloads' definitions):
  u, z, B, C, delta ~ N(0, 1), rounded to the input dtype (bf16: RNE);
  delta_bias[d] = log(expm1(U_d)), U_d ~ Uniform[1e-3, 1e-1] per channel,
      so softplus(delta + bias) equals U_d where delta = 0;
  D[d] ~ N(0, 1) per channel;
  A[d, n] = -(n + 1)                              ("s4d", S4D-real);
  A[d, n] = -(n + 1) * exp(eps_d), eps_d ~ N(0, 0.1) per row ("s4d_jitter");
  A[d, n] = -exp(A_log[d, n]), A_log = log(n + 1) + eps_d in fp32 ("alog": the
      same values up to the roundings of log and exp, which leave most rows
      without the exact (n + 1) A[d, 0] structure, as a trained A_log would);
  Mamba-2: A[h] = -U[1, 16], D[h] ~ N(0, 1), dt_bias as above, all per head.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# tensor ids of the per-tensor streams
_TID = {"u": 1, "delta": 2, "z": 3, "B": 4, "C": 5, "A": 6, "D": 7, "bias": 8, "dout": 9, "h0": 10}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "m1" or "m2"
    batch: int
    seqlen: int
    dstate: int
    dtype: torch.dtype   # u/delta/z/B/C (M2: x/dt/z/B/C)
    dim: int = 0         # M1 channels (d_inner)
    a_kind: str = "s4d"  # M1 A initialisation
    nheads: int = 0      # M2
    headdim: int = 0     # M2
    ngroups: int = 0     # M2
    note: str = field(default="", compare=False)
    out_dtype: torch.dtype = torch.float32   # y: fp32 (the state's precision)

    @property
    def updates(self) -> int:
        """State updates per scan: batch * L * channels * d_state."""
        ch = self.dim if self.kind == "m1" else self.nheads * self.headdim
        return self.batch * self.seqlen * ch * self.dstate


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "m1", batch=1, seqlen=64, dstate=16, dtype=torch.float32,
                          dim=32, a_kind="s4d",
                          note="tiny fp32 scan: batch 1, d_inner 32, d_state 16, L 64"),
    "mamba130m_l2k": Workload("mamba130m_l2k", "m1", batch=8, seqlen=2048, dstate=16,
                              dtype=torch.bfloat16, dim=1536, a_kind="s4d",
                              note="Mamba-130m-shaped layer: d_inner 1536, d_state 16, batch 8, L 2048"),
    "mamba2p8b_l8k": Workload("mamba2p8b_l8k", "m1", batch=4, seqlen=8192, dstate=16,
                              dtype=torch.bfloat16, dim=5120, a_kind="s4d_jitter",
                              note="Mamba-2.8b-shaped layer: d_inner 5120, d_state 16, batch 4, L 8192"),
    "long_1m": Workload("long_1m", "m1", batch=1, seqlen=1 << 20, dstate=16, dtype=torch.bfloat16,
                        dim=2048, a_kind="s4d_jitter",
                        note="million-token scan: d_inner 2048, d_state 16, batch 1, L 2^20"),
    "long_1m_shard8": Workload("long_1m_shard8", "m1", batch=1, seqlen=1 << 20, dstate=16, dtype=torch.bfloat16,
                               dim=256, a_kind="s4d_jitter",
                               note="one GPU's share of the million-token layer split 8 ways by channel: "
                                    "d_inner 256, d_state 16, batch 1, L 2^20"),
    "mamba2p8b_l8k_alog": Workload("mamba2p8b_l8k_alog", "m1", batch=4, seqlen=8192, dstate=16,
                                   dtype=torch.bfloat16, dim=5120, a_kind="alog",
                                   note="Mamba-2.8b-shaped layer with A = -exp(A_log) (no exact S4D-real "
                                        "structure: the general decay path)"),
    "mamba2_mh": Workload("mamba2_mh", "m2", batch=8, seqlen=4096, dstate=128, dtype=torch.bfloat16,
                          nheads=32, headdim=64, ngroups=1,
                          note="Mamba-2 multi-head: 32 heads x headdim 64, d_state 128, ngroups 1, "
                               "batch 8, L 4096"),
}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + _TID[name] * 7919) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _normal(shape, seed, name, dtype, device):
    dev = torch.device(device)
    out = torch.empty(shape, dtype=dtype, device=dev)
    g = _gen(seed, name, dev)
    # draw in fp32 and round once (RNE) to the storage dtype; chunked so the
    # fp32 temporary stays bounded for the multi-GB tensors
    flat = out.view(-1)
    step = 1 << 28
    for s in range(0, flat.numel(), step):
        e = min(flat.numel(), s + step)
        flat[s:e] = torch.randn(e - s, generator=g, device=dev, dtype=torch.float32).to(dtype)
    return out


def _cpu_uniform(n, lo, hi, seed, name):
    g = _gen(seed, name, "cpu")
    return torch.rand(n, generator=g, dtype=torch.float64) * (hi - lo) + lo


def delta_bias(n: int, seed: int) -> torch.Tensor:
    """bias = log(expm1(U)), U ~ Uniform[1e-3, 1e-1]; fp32 [n] on the CPU."""
    U = _cpu_uniform(n, 1e-3, 1e-1, seed, "bias")
    return torch.log(torch.expm1(U)).to(torch.float32)


def a_matrix(dim: int, dstate: int, kind: str, seed: int) -> torch.Tensor:
    n1 = torch.arange(1, dstate + 1, dtype=torch.float32)
    if kind == "s4d":
        return (-n1).repeat(dim, 1).contiguous()
    if kind == "s4d_jitter":
        g = _gen(seed, "A", "cpu")
        scale = torch.exp(torch.randn(dim, generator=g, dtype=torch.float32) * 0.1)
        return (-(n1[None, :] * scale[:, None])).contiguous()
    if kind == "alog":   # A = -exp(A_log), A_log = log(n + 1) + eps_d, both steps in fp32
        g = _gen(seed, "A", "cpu")
        eps = torch.randn(dim, generator=g, dtype=torch.float32) * 0.1
        a_log = torch.log(n1)[None, :] + eps[:, None]
        return (-torch.exp(a_log)).contiguous()
    if kind == "random":  # unstructured negative A, for the general decay path
        g = _gen(seed, "A", "cpu")
        return (-torch.rand(dim, dstate, generator=g, dtype=torch.float32) * 15.9 - 0.1).contiguous()
    raise ValueError(kind)


def m1_inputs(batch, dim, dstate, seqlen, dtype=torch.bfloat16, a_kind="s4d", seed=0,
              device="cpu", gate=True, skip=True, bias=True):
    """Inputs of one Mamba-1 scan as a dict of tensors.

    u, delta, z: [batch, dim, seqlen]; B, C: [batch, dstate, seqlen] (dtype);
    A: [dim, dstate], D, delta_bias: [dim] (fp32).
    """
    dev = torch.device(device)
    out = {
        "u": _normal((batch, dim, seqlen), seed, "u", dtype, dev),
        "delta": _normal((batch, dim, seqlen), seed, "delta", dtype, dev),
        "B": _normal((batch, dstate, seqlen), seed, "B", dtype, dev),
        "C": _normal((batch, dstate, seqlen), seed, "C", dtype, dev),
        "A": a_matrix(dim, dstate, a_kind, seed).to(dev),
        "z": _normal((batch, dim, seqlen), seed, "z", dtype, dev) if gate else None,
        "D": torch.randn(dim, generator=_gen(seed, "D", "cpu")).to(dev) if skip else None,
        "delta_bias": delta_bias(dim, seed).to(dev) if bias else None,
    }
    return out


def m1_row_sample(w: "Workload", rows: int, seed: int = 0):
    """The first `rows` channels of batch element 0 of a Mamba-1 workload, on
    the CPU, with the workload's distributions (a bounded sample for timing
    the CPU oracle on shapes too large for it)."""
    rows = max(1, min(rows, w.dim))
    cpu = torch.device("cpu")
    return {
        "u": _normal((1, rows, w.seqlen), seed, "u", w.dtype, cpu),
        "delta": _normal((1, rows, w.seqlen), seed, "delta", w.dtype, cpu),
        "B": _normal((1, w.dstate, w.seqlen), seed, "B", w.dtype, cpu),
        "C": _normal((1, w.dstate, w.seqlen), seed, "C", w.dtype, cpu),
        "A": a_matrix(w.dim, w.dstate, w.a_kind, seed)[:rows].contiguous(),
        "z": _normal((1, rows, w.seqlen), seed, "z", w.dtype, cpu),
        "D": torch.randn(w.dim, generator=_gen(seed, "D", "cpu"))[:rows].contiguous(),
        "delta_bias": delta_bias(w.dim, seed)[:rows].contiguous(),
    }


def m2_inputs(batch, seqlen, nheads, headdim, ngroups, dstate, dtype=torch.bfloat16, seed=0,
              device="cpu", gate=True, skip=True, bias=True):
    """Inputs of one Mamba-2 scan as a dict of tensors.

    x, z: [batch, seqlen, nheads, headdim]; dt: [batch, seqlen, nheads];
    B, C: [batch, seqlen, ngroups, dstate] (dtype); A, D, dt_bias: [nheads] fp32.
    """
    dev = torch.device(device)
    gA = _gen(seed, "A", "cpu")
    out = {
        "x": _normal((batch, seqlen, nheads, headdim), seed, "u", dtype, dev),
        "dt": _normal((batch, seqlen, nheads), seed, "delta", dtype, dev),
        "B": _normal((batch, seqlen, ngroups, dstate), seed, "B", dtype, dev),
        "C": _normal((batch, seqlen, ngroups, dstate), seed, "C", dtype, dev),
        "A": (-(torch.rand(nheads, generator=gA, dtype=torch.float32) * 15.0 + 1.0)).to(dev),
        "z": _normal((batch, seqlen, nheads, headdim), seed, "z", dtype, dev) if gate else None,
        "D": torch.randn(nheads, generator=_gen(seed, "D", "cpu")).to(dev) if skip else None,
        "dt_bias": delta_bias(nheads, seed).to(dev) if bias else None,
    }
    return out


def m1_dout(batch, dim, seqlen, dtype=torch.bfloat16, seed=0, device="cpu"):
    """Gradient of a loss with respect to a Mamba-1 scan's output: standard
    normal [batch, dim, seqlen], drawn like the inputs."""
    return _normal((batch, dim, seqlen), seed, "dout", dtype, torch.device(device))


def m2_dout(batch, seqlen, nheads, headdim, dtype=torch.float32, seed=0, device="cpu"):
    """Gradient of a loss with respect to a Mamba-2 scan's output: standard
    normal [batch, seqlen, nheads, headdim], drawn like the inputs."""
    return _normal((batch, seqlen, nheads, headdim), seed, "dout", dtype, torch.device(device))


def m2_state(batch, nheads, headdim, dstate, seed=0, device="cpu"):
    """A Mamba-2 state [batch, nheads, headdim, dstate] fp32, standard normal."""
    return _normal((batch, nheads, headdim, dstate), seed, "h0", torch.float32, torch.device(device))


def m1_state(batch, dim, dstate, seed=0, device="cpu"):
    """A Mamba-1 state [batch, dim, dstate] fp32, standard normal."""
    return _normal((batch, dim, dstate), seed, "h0", torch.float32, torch.device(device))


def bwd_algorithmic_bytes(w: Workload) -> int:
    """Bytes the backward must move: the forward's inputs and dout (of the
    output's dtype) read once, every fp32 gradient written once."""
    s = torch.tensor([], dtype=w.dtype).element_size()
    so = torch.tensor([], dtype=w.out_dtype).element_size()
    if w.kind == "m2":
        elem = w.batch * w.seqlen * w.nheads * w.headdim
        tok = w.batch * w.seqlen * w.nheads
        bc = w.batch * w.seqlen * w.ngroups * w.dstate
        return (elem * (2 * s + so) + tok * s + 2 * bc * s + 3 * w.nheads * 4
                + elem * 2 * 4 + tok * 4 + 2 * bc * 4 + 3 * w.nheads * 4)
    elem = w.batch * w.dim * w.seqlen
    bc = w.batch * w.dstate * w.seqlen
    return (elem * (3 * s + so) + 2 * bc * s + (w.dim * w.dstate + 2 * w.dim) * 4
            + elem * 3 * 4 + 2 * bc * 4 + (w.dim * w.dstate + 2 * w.dim) * 4)


def workload_inputs(w: Workload | str, seed: int = 0, device="cpu"):
    if isinstance(w, str):
        w = WORKLOADS[w]
    if w.kind == "m1":
        return m1_inputs(w.batch, w.dim, w.dstate, w.seqlen, w.dtype, w.a_kind, seed, device)
    return m2_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate, w.dtype, seed,
                     device)


def algorithmic_bytes(w: Workload) -> int:
    """Bytes the scan must move: every input read once, y and the final state
    written once, no intermediate state."""
    s = torch.tensor([], dtype=w.dtype).element_size()
    so = torch.tensor([], dtype=w.out_dtype).element_size()
    if w.kind == "m1":
        elem = w.batch * w.dim * w.seqlen
        return (elem * (3 * s + so) + 2 * w.batch * w.dstate * w.seqlen * s
                + (w.dim * w.dstate + 2 * w.dim) * 4 + w.batch * w.dim * w.dstate * 4)
    elem = w.batch * w.seqlen * w.nheads * w.headdim
    return (elem * (2 * s + so) + w.batch * w.seqlen * w.nheads * s
            + 2 * w.batch * w.seqlen * w.ngroups * w.dstate * s + 3 * w.nheads * 4
            + w.batch * w.nheads * w.headdim * w.dstate * 4)


__all__ = ["WORKLOADS", "Workload", "m1_inputs", "m1_row_sample", "m2_inputs", "workload_inputs",
           "algorithmic_bytes", "bwd_algorithmic_bytes", "a_matrix", "delta_bias", "m1_dout", "m1_state"]
