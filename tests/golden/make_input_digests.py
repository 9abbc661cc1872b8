"""Write input_digests.json: SHA-256 of the synthetic inputs of the small workloads.

This pins the input recipe (generator, seed, draw order, distribution and
bf16 rounding) across machines and library versions. It calls only the input
generator; no GEMM result is involved.

Run from the repository root: python tests/golden/make_input_digests.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from tiled_dense_matrix_amd import inputs  # noqa: E402

NAMES = ["f32_256", "bf16_skinny"]


def main():
    out = {}
    for name in NAMES:
        A, B = inputs.make_inputs(name)
        out[name] = {"A": inputs.digest(A), "B": inputs.digest(B)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_digests.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=2, sort_keys=True)
        fh.write("\n")
    print(path)


if __name__ == "__main__":
    main()
