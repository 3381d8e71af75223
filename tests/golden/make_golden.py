"""Writes tiny_mha_seed1.txt: the oracle's outputs for the tiny MHA workload (seed 1).

Calls only the oracle (and the seeded input generator).  The file freezes the oracle so that an
unintended change to its arithmetic shows up as a test failure; a deliberate change regenerates
it and names, in its commit message, the passage of the pages or the reading that justifies it.
Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import synth  # noqa: E402
from oracle_pipeline import oracle_step  # noqa: E402


def render():
    w = synth.make("tiny_mha", seed=1)
    r = oracle_step(w, "fp8")
    lines = ["# oracle outputs, tiny MHA workload (B4, L {17,64,129,200}, 8/8 heads, D64, P16, 64 pages), seed 1"]
    lines.append("k_scale " + " ".join(float(x).hex() for x in r["k_scale"]))
    lines.append("v_scale " + " ".join(float(x).hex() for x in r["v_scale"]))
    lines.append("k_pool_sha256 " + hashlib.sha256(r["k_pool"].tobytes()).hexdigest())
    lines.append("v_pool_sha256 " + hashlib.sha256(r["v_pool"].tobytes()).hexdigest())
    lines.append("abort " + " ".join(str(int(x)) for x in r["abort"]))
    out = r["out"]
    for b in range(out.shape[0]):
        for h in range(out.shape[1]):
            lines.append(f"out {b} {h} " + " ".join(float(x).hex() for x in out[b, h]))
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_mha_seed1.txt")
    with open(path, "w") as f:
        f.write(render())
    print("wrote", path)
