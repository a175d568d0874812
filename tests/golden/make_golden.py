"""Write tests/golden/oracle_workload0.json: fp64 oracle outputs on the seeded
tiny workload (M=16, H=256, V=4096, 4-bit), the regression fixture that
tests/test_golden.py checks the oracle (CPU) and the HIP path (GPU) against.

Calls only the oracle; run from the repository root:
    python3 tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "oracle"))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from linear_cross_entropy_libcce_amd import synthetic as syn  # noqa: E402

DH_TOKENS = [0, 5, 11, 15]   # rows of dh stored (all of logp and lse are)


def main():
    inp = syn.make_inputs(syn.WORKLOADS[0], syn.seed_for(0))
    g = np.linspace(-1.0, 1.0, inp["M"])
    logp, lse, dh = oracle.cce(inp, g=g)
    out = {
        "about": "fp64 oracle outputs for synthetic workload 0 (seed %d), g = linspace(-1, 1, M); "
                 "written by tests/golden/make_golden.py" % syn.seed_for(0),
        "workload": 0, "seed": syn.seed_for(0), "M": inp["M"], "H": inp["H"], "V": inp["V"], "bits": inp["bits"],
        "g": [float(x) for x in g],
        "logp": [float(x) for x in logp],
        "lse": [float(x) for x in lse],
        "dh_tokens": DH_TOKENS,
        "dh": [[float(x) for x in dh[t]] for t in DH_TOKENS],
    }
    path = os.path.join(ROOT, "tests", "golden", "oracle_workload0.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
