"""Writes the small fixtures in this folder.

Inputs are drawn with numpy (seeded) and rounded to fp32; the expected
outputs come from the fp64 oracle only (``oracle.m1`` / ``oracle.m2``), never
from the HIP library.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402


def _f32(a):
    return np.asarray(a, np.float32).astype(np.float64)


def m1_case():
    rng = np.random.default_rng(2024)
    nb, nd, nn, nl = 2, 3, 4, 13
    x = dict(u=_f32(rng.standard_normal((nb, nd, nl))), delta=_f32(rng.standard_normal((nb, nd, nl))),
             A=_f32(-np.tile(np.arange(1, nn + 1), (nd, 1)) * np.exp(0.1 * rng.standard_normal((nd, 1)))),
             B=_f32(rng.standard_normal((nb, nn, nl))), C=_f32(rng.standard_normal((nb, nn, nl))),
             D=_f32(rng.standard_normal(nd)), z=_f32(rng.standard_normal((nb, nd, nl))),
             delta_bias=_f32(np.log(np.expm1(rng.uniform(1e-3, 1e-1, nd)))))
    y, last = oracle.m1(**x, softplus=True)
    return {"kind": "m1", "softplus": True,
            "inputs": {k: v.tolist() for k, v in x.items()},
            "y": y.tolist(), "last_state": last.tolist()}


def m2_case():
    rng = np.random.default_rng(2025)
    nb, nl, nh, npd, ng, nn = 1, 9, 4, 2, 2, 16
    x = dict(x=_f32(rng.standard_normal((nb, nl, nh, npd))), dt=_f32(rng.standard_normal((nb, nl, nh))),
             A=_f32(-rng.uniform(1, 16, nh)), B=_f32(rng.standard_normal((nb, nl, ng, nn))),
             C=_f32(rng.standard_normal((nb, nl, ng, nn))), D=_f32(rng.standard_normal(nh)),
             z=_f32(rng.standard_normal((nb, nl, nh, npd))),
             dt_bias=_f32(np.log(np.expm1(rng.uniform(1e-3, 1e-1, nh)))))
    y, last = oracle.m2(**x, softplus=True)
    return {"kind": "m2", "softplus": True,
            "inputs": {k: v.tolist() for k, v in x.items()},
            "y": y.tolist(), "last_state": last.tolist()}


def main():
    for name, fn in (("m1_small.json", m1_case), ("m2_small.json", m2_case)):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fn(), f, indent=None, separators=(",", ":"))
            f.write("\n")


if __name__ == "__main__":
    main()
