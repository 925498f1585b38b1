"""Write the oracle regression fixtures in this folder.

The pages print no worked numeric example for the skinny linear, so these
fixtures are not page values: they freeze the oracle's own outputs on small
seeded inputs, so that any later change to the oracle's arithmetic shows up as
a test failure and has to be justified.  Only ``oracle`` and ``synth`` are
called.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synth  # noqa: E402

CASES = [(4, 2, 8, 256), (6, 3, 8, 256)]


def compute():
    out = []
    for bits, M, N, K in CASES:
        canon, S = synth.weights(bits, N, K, seed=77)
        x = synth.activations(M, K, seed=78)
        q, s = oracle.quantize_act(x)
        acc = oracle.group_acc(bits, q, canon)
        y = oracle.linear(bits, q, s, canon, S)
        t = oracle.rmsnorm_bf16(x)
        out.append(dict(bits=bits, M=M, N=N, K=K, weight_seed=77, act_seed=78,
                        s=[float(v) for v in s], q_sum=[int(v) for v in q.astype(int).sum(axis=1)],
                        acc=acc.reshape(-1).tolist(), y=[int(v) for v in y.reshape(-1)],
                        rmsnorm_t_head=[int(v) for v in t[:, :16].reshape(-1)]))
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(compute(), f, indent=0)
        f.write("\n")
