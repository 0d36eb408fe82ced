"""Writes tiny_bruteforce.json: a small bf16 case scored by the brute-force oracle.

The expected values come only from ``oracle.brute`` (exact rational logits and
50-digit decimal exp/ln); they are stored to 30 significant digits. Run from
the repository root:  python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import brute, decode_bf16  # noqa: E402

T, H, V = 5, 12, 48


def main():
    r = np.random.default_rng(2024)
    h = torch.from_numpy(r.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    # logits of spread ~3 so entropies range from peaky to broad
    W = torch.from_numpy((r.standard_normal((V, H)) * 0.9).astype(np.float32)).to(torch.bfloat16)
    y = r.integers(0, V, T)
    hb = h.view(torch.int16).numpy().view(np.uint16)
    Wb = W.view(torch.int16).numpy().view(np.uint16)
    logp, ent = brute.logp_entropy(decode_bf16(hb), decode_bf16(Wb), y)
    out = {
        "about": "brute-force (exact rationals + 50-digit decimal) logp/entropy of a tiny bf16 case",
        "T": T, "H": H, "V": V,
        "hidden_bits": hb.reshape(-1).tolist(),
        "weight_bits": Wb.reshape(-1).tolist(),
        "targets": y.tolist(),
        "logp": [f"{x:.30g}" for x in logp],
        "entropy": [f"{x:.30g}" for x in ent],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_bruteforce.json")
    with open(path, "w") as f:
        json.dump(out, f)
    print("wrote", path)


if __name__ == "__main__":
    main()
