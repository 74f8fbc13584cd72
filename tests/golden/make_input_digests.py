"""Writes input_digests.json: the SHA-256 of every workload's generated input
(data seed 0).  Calls only the input generator, never the oracle or the GPU
path; the digests pin the generator so that stored expectations and the
benchmark keep seeing the same tensors."""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import workloads  # noqa: E402


def main() -> None:
    out = {}
    for k, c in workloads.CONFIGS.items():
        x = workloads.inputs(c, seed=0)
        out[str(k)] = {"name": c["name"], "shape": list(x.shape), "dtype": str(x.dtype), "sha256": workloads.digest(x)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_digests.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
