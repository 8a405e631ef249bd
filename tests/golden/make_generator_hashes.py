"""Writes generator_sha256.json: SHA-256 of a few generator outputs (a regression
pin of the input streams, not a correctness pin). Calls only attn_inputs."""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import attn_inputs as ai  # noqa: E402

CASES = {
    "slab_q_seed1_b0_h0_128x64_bf16": ("slab", 1, ai.Q_ID, 0, 0, 128, 64, ai.BF16),
    "slab_k_seed2_b1_h7_64x64_fp16": ("slab", 2, ai.K_ID, 1, 7, 64, 64, ai.FP16),
    "slab_v_seed3_b0_h3_32x128_bf16": ("slab", 3, ai.V_ID, 0, 3, 32, 128, ai.BF16),
    "lengths_seed5_b32": ("lengths", 5, 32, 1024, 32768),
}


def digest(kind, *args):
    if kind == "slab":
        data = ai.slab(*args)
    else:
        data = ai.decode_lengths(*args)
    return hashlib.sha256(data.tobytes()).hexdigest()


if __name__ == "__main__":
    out = {name: digest(*args) for name, args in CASES.items()}
    with open(os.path.join(HERE, "generator_sha256.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(out)
