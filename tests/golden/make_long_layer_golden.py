"""Write the oracle's values of the B=8, N=32768, d=1024 bf16 layer at sampled
positions of one batch row (tests/golden/long_d1024_b8_n32768_row0.npz).

The oracle (oracle/rt_oracle.c, the naive schedule with bf16 storage
emulation) takes minutes for one row of all 32768 positions, too long for a
test, so its values at the sampled positions are stored: z, k, v before their
own rounding, as float32. Batch rows are independent, so the row's values
are those of the full 8-row layer. Inputs are the workload's own seeded draws
(rt_inputs, workload long_d1024_b8_n32768): x row 0 and the layer's weights,
gains of ones, softmax scale 1/sqrt(64), residual scale 1.

Run from the repository root:  python tests/golden/make_long_layer_golden.py
"""
import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import rt_inputs  # noqa: E402

ROW = 0
POSITIONS = [1, 2, 3, 1024, 1025, 2048, 2049, 4096, 4097, 8192, 8193, 16384, 16385, 24576, 32767, 32768]
OUT = os.path.join(HERE, "long_d1024_b8_n32768_row0.npz")


def main():
    wl = rt_inputs.WORKLOADS["long_d1024_b8_n32768"]
    x = rt_inputs.layer_input(wl, rows=[ROW])
    w = rt_inputs.layer_weights(wl, 0)
    t0 = time.time()
    ref = oracle.layer_forward(x, w, n_heads=wl.n_heads, softmax_scale=1.0 / math.sqrt(wl.head_dim),
                               round_bf16=True)
    sel = np.array(POSITIONS) - 1
    np.savez(OUT, positions=np.array(POSITIONS, dtype=np.int32),
             **{n: ref[n][sel, 0].astype(np.float32) for n in ("z", "k", "v")})
    meta = {"workload": wl.name, "row": ROW, "positions": POSITIONS, "oracle_seconds": round(time.time() - t0, 1),
            "threads": oracle.num_threads(), "made_by": "python tests/golden/make_long_layer_golden.py"}
    with open(OUT.replace(".npz", ".json"), "w") as f:
        json.dump(meta, f, indent=1)
    print(json.dumps(meta))


if __name__ == "__main__":
    main()
