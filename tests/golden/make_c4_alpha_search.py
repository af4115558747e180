"""Write tests/golden/c4_alpha_search_oracle.json: the oracle's alpha grid
search on the full alpha-search workload (8 calibration batches of 2048
tokens, Student-t nu = 3 activations with 12 outlier channels x 50, K = 4096,
N = 11008; ADR-010 "Key design" item 2: a full W8A8 forward per alpha in the
grid {0.25, 0.5, 0.75, 1.0}, the error against the unquantized product, the
argmin). Calls only oracle/ on the seeded inputs of synth.py; takes a few
minutes on a few cores. The file records a digest of the inputs so a change to
the input recipe is caught instead of compared against stale values.

    python tests/golden/make_c4_alpha_search.py
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c4_alpha_search_oracle.json")


def input_digest(xs, w) -> str:
    h = hashlib.sha256()
    for a in list(xs) + [w]:
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


def main() -> None:
    from oracle.oracle import Oracle
    from w8a8_post_quantization_channel_amd import synth

    xs = synth.c4_batches(8)
    w = synth.c4_weight()
    t = time.time()
    o = Oracle()
    mse, best = o.alpha_search(xs, w)
    rec = {
        "source": "ADR-010 'SmoothQuant Integration', Key design item 2 (per-layer alpha grid search)",
        "workload": "8 x 2048 tokens, K = 4096 -> N = 11008, synth.c4_batches(8) / synth.c4_weight()",
        "alphas": [0.25, 0.5, 0.75, 1.0],
        "mse": [float(v) for v in mse],
        "mse_hex": [float(v).hex() for v in mse],
        "best": int(best),
        "input_sha256": input_digest(xs, w),
        "oracle_threads": o.num_threads(),
        "oracle_seconds": round(time.time() - t, 1),
    }
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
