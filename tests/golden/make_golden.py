"""Write tests/golden/tiny_oracle.txt: the oracle's result on the Tiny workload.

Tiny workload: hidden 256, intermediate 512, 8 experts, top-2, 16 tokens,
x ~ N(0,1), weights ~ N(0,0.02), router logits ~ N(0,1), seed 0 (drawn by
workloads.py on the CPU).  This script calls only ``oracle/`` and
``workloads.py``; no value in the file comes from the HIP library.  The file
is a regression record: a later change of oracle arithmetic or of the input
recipe shows up as a mismatch, and the commit that regenerates the file must
name the passage or reading that justifies the change.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(HERE, "tiny_oracle.txt")


def compute():
    wl = workloads.WORKLOADS["tiny"]
    x = workloads.bf16_bits(workloads.gen_x(wl))
    ids, w = oracle.route_topk(workloads.gen_logits(wl).numpy(), wl.k)
    Wg, Wu, Wd = (workloads.bf16_bits(t) for t in workloads.gen_weights(wl, "cpu"))
    out = oracle.moe_ffn_bf16(x, ids, w, Wg, Wu, Wd, E=wl.E)
    return ids, w, out


def main():
    ids, w, out = compute()
    with open(OUT, "w") as f:
        f.write("# Oracle result, Tiny MoE FFN workload (H256 I512 E8 top-2 T16 seed0).\n")
        f.write("# Written by tests/golden/make_golden.py (oracle only).\n")
        f.write("# ids: token expert ids; w: routing weights as float32 hex; out: bf16 hex rows\n")
        for t in range(ids.shape[0]):
            f.write("ids " + " ".join(str(int(v)) for v in ids[t]) + "\n")
            f.write("w " + " ".join(f"{int(v):08x}" for v in w[t].view(np.uint32)) + "\n")
            f.write("out " + " ".join(f"{int(v):04x}" for v in out[t]) + "\n")
    print(OUT)


def load():
    ids, w, out = [], [], []
    for line in open(OUT):
        if line.startswith("#"):
            continue
        tag, *vals = line.split()
        if tag == "ids":
            ids.append([int(v) for v in vals])
        elif tag == "w":
            w.append(np.array([int(v, 16) for v in vals], np.uint32).view(np.float32))
        elif tag == "out":
            out.append([int(v, 16) for v in vals])
    return (np.array(ids, np.int32), np.array(w, np.float32),
            np.array(out, np.uint16))


if __name__ == "__main__":
    main()
