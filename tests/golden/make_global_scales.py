"""Write global_scales.json: the static NVFP4 global scale of each workload's
pre-expert norm input, 448 * 6 / amax of the normalised tensor.

Calls only the oracle and the seeded input generators:
    python tests/golden/make_global_scales.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O          # noqa: E402
import workloads as wl      # noqa: E402


def amax_normalised(w, chunk=1024):
    x = wl.quant_input(w)
    nw = wl.quant_gain(w)
    amax = 0.0
    for r0 in range(0, w.T, chunk):
        y = O.rmsnorm_bf16(x[r0:r0 + chunk], nw, w.quant_gain_center, w.eps)
        amax = max(amax, float(np.max(np.abs(y))))
    return amax


def main():
    out = {}
    for name, w in wl.WORKLOADS.items():
        amax = amax_normalised(w)
        gs = O.global_scale(np.array([amax], dtype=np.float32))
        out[name] = {"amax": amax, "global_scale": float(gs), "global_scale_hex": float(gs).hex()}
        print(name, out[name])
    with open(os.path.join(HERE, "global_scales.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
