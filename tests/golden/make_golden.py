"""Write tests/golden/tiny_2of4_seed0.json from the CPU oracle alone.

Regression fixture for the tiny workload (W 256x512 bf16 ~ 0.02 N(0,1), 16 calibration
tokens with lognormal channel scales, 2:4, x ~ N(0,1), seed 0).  The pages print no
worked numbers for this case; the digests here were produced by the oracle and only
guard against silent changes to it or to the input generators.

Run:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

R, K, N, M, SEED = 256, 512, 2, 4, 0


def tiny_inputs():
    W = synth.weights(R, K, SEED)
    X = synth.calib_acts(K, SEED)
    x = synth.decode_x(1, K, SEED)
    return W, X, x


def digest(a) -> str:
    return hashlib.sha256(a.tobytes()).hexdigest()


def main():
    W, X, x = tiny_inputs()
    n = oracle.col_norm(X)
    masks, values = oracle.prune_pack(W, n, N, M)
    y, a = oracle.spmv(masks, values, x, K)
    yd, _ = oracle.dense(W, x)
    out = {
        "workload": "tiny: W 256x512 bf16, 2:4, B=1, seed 0",
        "sha256_W": digest(W), "sha256_X": digest(X), "sha256_x": digest(x),
        "sha256_col_norm": digest(n), "sha256_masks": digest(masks), "sha256_values": digest(values),
        "sha256_y_ref": digest(y), "sha256_y_dense_ref": digest(yd),
        "y_ref_head": [float(v).hex() for v in y[0, :8]],
        "mask_row0_head": [int(v) for v in masks[0, :4]],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_2of4_seed0.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
