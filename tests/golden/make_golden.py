"""Write tests/golden/tiny_oracle_digest.json from the oracle alone.

The digest freezes the oracle's quantizer output on the tiny outlier workload (seed 0) so
that an unintended change to the oracle's arithmetic shows up as a test failure;
a deliberate change re-runs this script and names the passage that justifies it
in the commit message.  Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import quant  # noqa: E402
from workloads import draw  # noqa: E402


def digest():
    d = draw("tiny")
    qx, sx = quant.quant_act_1x128(d["X"])
    qw, sw, qwT, swT = quant.quant_w_128x128(d["W"])
    h = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    return {
        "workload": "tiny (seed 0): X 256x512 N(0,1) with 0.5% x20 outliers, W 384x512 N(0,0.02)",
        "X_bits_sha256": h(d["X"]), "W_bits_sha256": h(d["W"]),
        "qX_sha256": h(qx), "sX_sha256": h(sx),
        "qW_sha256": h(qw), "sW_sha256": h(sw), "qWT_sha256": h(qwT), "sWT_sha256": h(swT),
        "sX_first": [float(v) for v in sx[0, :4]], "sW": [[float(v) for v in r] for r in sw],
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_digest.json")
    with open(out, "w") as f:
        json.dump(digest(), f, indent=1)
    print("wrote", out)
