"""Write tests/golden/input_checksums.json: SHA-256 of the seeded inputs.

The digests freeze the input generator (causal_flash_attention_amd.inputs) so
that a change to its definition shows up as a test failure. Run from the
repository root: python tests/golden/make_input_checksums.py
"""

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from causal_flash_attention_amd import inputs  # noqa: E402
from causal_flash_attention_amd.workloads import WORKLOADS  # noqa: E402


def digests():
    out = {}
    for w in WORKLOADS:
        if w.B * w.T * w.C * 4 > 200_000_000:
            continue
        qkv, dout = inputs.attention_inputs(w.B, w.T, w.n_head, w.head_dim, w.dtype,
                                            w.qkv_std, w.dout_std, seed=0)
        out[w.name] = {"qkv": hashlib.sha256(qkv.tobytes()).hexdigest(),
                       "dout": hashlib.sha256(dout.tobytes()).hexdigest()}
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "input_checksums.json"), "w") as f:
        json.dump(digests(), f, indent=1, sort_keys=True)
        f.write("\n")
