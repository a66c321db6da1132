"""Write input_digests.txt: the SHA-256 of every buffer the seeded generator produces for each
named workload (A, B, then C and the 2:4 metadata where the workload has them), so that a
change to the generator or to numpy's PCG64 stream shows up as a failing test.  Calls only
gemm_inputs."""
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from gemm_inputs import NEXT_WORKLOADS, WORKLOADS, generate  # noqa: E402


def digests(name, w):
    inp = generate(w)
    out = []
    for label in ("A", "B", "C", "meta"):
        arr = getattr(inp, label, None)
        if arr is None:
            continue
        h = hashlib.sha256(arr.tobytes()).hexdigest()
        out.append(f"{name} {label} {arr.dtype} {'x'.join(map(str, arr.shape))} {h}")
    return out


def main():
    lines = ["# workload buffer dtype shape sha256 (written by make_input_digests.py)"]
    for table in (WORKLOADS, NEXT_WORKLOADS):
        for name, w in table.items():
            lines += digests(name, w)
    with open(os.path.join(HERE, "input_digests.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
