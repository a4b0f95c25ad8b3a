"""Writes rope_hd4.json: RoPE of a few 4-dim vectors as complex rotations.

Closed form only (no oracle): with head dim 4 and base theta, pair k couples
components k and k+2 and turns them by pos / theta^(2k/4), the rotate-half
pairing of HF apply_rotary_pos_emb that the DeepSpec drafter page says its
port was checked against (deepspec.ts header; #projectContextKVRows rope).
"""
import cmath
import json
import os

THETA = 10000.0
CASES = [([1.0, 0.0, 0.0, 0.0], 1), ([0.0, 1.0, 0.0, 0.0], 1), ([0.5, -2.0, 1.5, 3.0], 7),
         ([1.0, 1.0, 1.0, 1.0], 100), ([-1.25, 0.75, 2.0, -0.5], 32768)]


def rotate(x, pos):
    y = [0.0] * 4
    for k in range(2):
        z = complex(x[k], x[k + 2]) * cmath.exp(1j * pos / THETA ** (2 * k / 4))
        y[k], y[k + 2] = z.real, z.imag
    return y


if __name__ == "__main__":
    out = {"head_dim": 4, "theta": THETA,
           "source": "closed form: complex rotation of pairs (k, k+2) by pos/theta^(2k/4)",
           "cases": [{"x": x, "pos": p, "y": rotate(x, p)} for x, p in CASES]}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "rope_hd4.json"), "w") as f:
        json.dump(out, f, indent=1)
