"""Write the oracle's outputs for the tiny decode workload to a fixture.

Calls only ``oracle`` (and the seeded generators in ``workloads``).  The pages
print no worked example for any step of the path, so this fixture is a
regression anchor for the oracle itself, not an independent pin: a later
change to the oracle's arithmetic that moves these values must say which
passage, or which reading of it, justifies the change.

Run from the repository root:  python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from workloads import CONFIGS, make_batch, oracle_arrays  # noqa: E402


def compute():
    wl = CONFIGS["tiny_decode_1x1k"]
    arr = oracle_arrays(make_batch(wl, device="cpu", seed=wl.seed))
    res = oracle.decode_step(
        qI=arr["qI"], w=arr["w"], kI_cache=arr["kI_cache"], q=arr["q"],
        k_cache=arr["k_cache"], v_cache=arr["v_cache"], block_table=arr["block_table"],
        seq_lens=arr["seq_lens"], K=arr["K"], scale=arr["scale"], D_v=arr["D_v"])
    scores = res["scores"][0]
    return {
        "workload": wl.name, "seed": wl.seed, "mode": wl.mode,
        "count": int(res["counts"][0]),
        "indices": res["indices"][0].tolist(),
        "scores_sha256": hashlib.sha256(scores.astype("<f4").tobytes()).hexdigest(),
        "scores_first8": [float(x) for x in scores[:8]],
        "score_max": float(scores.max()),
        "out_head0_first8": [round(float(x), 12) for x in res["out"][0, 0, :8]],
        "lse": [round(float(x), 12) for x in res["lse"][0]],
    }


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_decode_1x1k_seed1.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=1)
        f.write("\n")
    print("wrote", path)
