"""Write tests/golden/hashes.json: SHA-256 of the oracle's bit-exact outputs.

Fixed-token, hash-based correctness checks are how the paper pins its
corrected path before optimising ("DeepSeek-V4-Flash on AMD gfx90a:
Correctness Recovery and Inference Performance Engineering", abstract).
Calls only ``synth`` (inputs) and ``oracle`` (values).  Run from the repo root:
    python tests/golden/make_hashes.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def bit_exact_outputs(name: str) -> dict:
    inp = synth.make_inputs(name, with_weights=False)
    sh = inp.shape
    ids, _ = oracle.route(inp.logits, sh.k)
    counts, offsets, sp, pp = oracle.sort(ids, sh.E)
    xq, xs = oracle.quant_mxfp8_bf16(inp.x)
    return {"topk_ids": ids, "expert_counts": counts, "expert_offsets": offsets,
            "sorted_pair": sp, "pair_pos": pp, "xq": xq, "xs": xs}


def main():
    out = {}
    for name in synth.CONFIGS:
        out[name] = {k: sha(v) for k, v in bit_exact_outputs(name).items()}
        print(name, "done", flush=True)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "hashes.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
