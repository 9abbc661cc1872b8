"""Write input_digests.json: SHA-256 of the synthetic inputs of every workload.

This pins the input recipe (generator, seed, draw order, distribution, bf16
rounding, FP8 block quantization) across machines and library versions. It
calls only the input generator; no product or other result of the method is
involved.

Run from the repository root: python tests/golden/make_input_digests.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from tiled_dense_matrix_amd import inputs  # noqa: E402


def workload_digests(name: str) -> dict:
    """Digests of one workload's arrays, keyed by what they are."""
    if name in inputs.ATTN_WORKLOADS:
        Q, K, V = inputs.make_attention_inputs(name)
        return {"Q": inputs.digest(Q), "K": inputs.digest(K), "V": inputs.digest(V)}
    w = inputs.WORKLOADS[name]
    if w.kind == "fp8":
        A, B, sa, sb = inputs.make_fp8_inputs(w)
        out = {"A": inputs.digest(A), "B": inputs.digest(B)}
        if sa is not None:
            out["a_scale"] = inputs.digest(sa)
            out["b_scale"] = inputs.digest(sb)
        return out
    A, B = inputs.make_inputs(w)
    out = {"A": inputs.digest(A), "B": inputs.digest(B)}
    if w.bias_sigma > 0:
        out["bias"] = inputs.digest(inputs.make_bias(w))
    return out


def names():
    return sorted(inputs.WORKLOADS) + sorted(inputs.ATTN_WORKLOADS)


def main():
    out = {name: workload_digests(name) for name in names()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_digests.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=2, sort_keys=True)
        fh.write("\n")
    print(path)


if __name__ == "__main__":
    main()
