"""Writes the stored fixtures under tests/golden/.  Calls only the seeded
generator (workload/) and the CPU oracle (oracle/); never the GPU path.

  input_digests.json  sha256 of every generated buffer for a few small ad-hoc
                      problems and the five configurations -- pins "same seed,
                      same bytes" across machines and library versions.
  oracle_cfg1.json    oracle O/LSE on sampled rows of configuration 1 (regression
                      pin for the oracle itself; a change here must name the
                      passage or reading that justifies it).

Run from the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workload as W  # noqa: E402
import oracle  # noqa: E402

SMALL_SPECS = {
    "tiny_bf16": dict(B=1, H=2, N=65, d=64, seed=1),
    "doc_bf16": dict(B=2, H=1, N=300, d=128, flags=W.ATTN_CAUSAL | W.ATTN_DOCUMENT, seed=2),
    "fp8": dict(B=1, H=2, N=200, d=128, dtype="fp8", n_outliers=4, seed=3),
}


def main():
    small = {name: W.make_problem(**spec).digests() for name, spec in SMALL_SPECS.items()}
    configs = {str(c): W.config_problem(c).digests() for c in range(1, 6)}
    with open(os.path.join(HERE, "input_digests.json"), "w") as f:
        json.dump({"small_specs": SMALL_SPECS, "small": small, "configs": configs}, f, indent=1,
                  sort_keys=True)
        f.write("\n")

    p = W.config_problem(1)
    rows = np.array([0, 1, 2, 63, 64, 127, 128, 200, 254, 255])
    o, lse = oracle.attention_problem(p, rows=rows)
    with open(os.path.join(HERE, "oracle_cfg1.json"), "w") as f:
        json.dump({"rows": rows.tolist(), "O": o.tolist(), "LSE": lse.tolist()}, f)
        f.write("\n")


if __name__ == "__main__":
    main()
