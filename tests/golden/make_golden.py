"""Write the stored oracle outputs for the 27-layer workloads.

Calls only oracle/ (float64 CPU oracle) and synthetic/ (seeded inputs):
  oracle_c3_27layer_seed1.npz   images 0 and 1 of seed 1 (F16-path configs,
                                B=1 uses image 0, B=2 both)
  oracle_c4_27layer_seed2.npz   images 0, 21, 42, 63 of the B=64 seed-2 batch,
                                unquantized (the accuracy bar of the FP8 path)
                                and with e4m3 operands (diagnostic)
Each file also stores checksums of the generated inputs, so a test can tell
a changed random stream from a wrong kernel.

Run: python tests/golden/make_golden.py   (a few minutes on 8 cores)
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
import synthetic as S  # noqa: E402


def input_checksums(wt, pixels):
    return np.array([float(np.sum(pixels, dtype=np.float64)),
                     float(np.sum(wt["embed.w"], dtype=np.float64)),
                     float(np.sum(wt["layer26.mlp2.w"], dtype=np.float64)),
                     float(np.sum(wt["map.mlp2.w"], dtype=np.float64))])


def main():
    d = S.SO400M
    wt = S.make_weights(d, 1)
    x = S.make_pixels(d, 2, 1)
    y = O.encode(wt, x, d.heads)
    np.savez(os.path.join(HERE, "oracle_c3_27layer_seed1.npz"), images=np.array([0, 1]),
             out=y[:, 0, :], checksums=input_checksums(wt, x))
    print("c3 done", np.abs(y).max())

    wt = S.make_weights(d, 2)
    idx = np.array([0, 21, 42, 63])
    x = S.make_pixels(d, 64, 2)
    xs = x[idx]
    y = O.encode(wt, xs, d.heads)
    y8 = O.encode(wt, xs, d.heads, fp8=True)
    np.savez(os.path.join(HERE, "oracle_c4_27layer_seed2.npz"), images=idx, out=y[:, 0, :],
             out_fp8_operands=y8[:, 0, :], checksums=input_checksums(wt, x))
    print("c4 done", np.abs(y).max(), np.abs(y - y8).max())


if __name__ == "__main__":
    main()
