"""Write the stored outputs of the fixture workload (batch 2, 512 tokens,
4 heads x 16 dims, indexer 4 x 16, top-32, window 16, fp32).

The pages print no worked example, so no stored value here comes from them:
every number below is written by this script, which calls only the CPU oracle
(on inputs from the shared seeded generator).  The file guards the oracle's
arithmetic against unnoticed change; it does not pin it.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from compressed_sparse_attention_indexer_amd import inputs  # noqa: E402


def main():
    case = inputs.make_case(inputs.WORKLOADS["fixture_b2_l512_fp32"])
    scores, idx, out, lse = oracle.csa_attention(case)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fixture_b2_l512_fp32.json")
    with open(path, "w") as f:
        json.dump({"workload": "fixture_b2_l512_fp32",
                   "written_by": "tests/golden/make_golden.py (CPU oracle only)",
                   "scores": scores.tolist(), "topk_idx": idx.tolist(),
                   "out": out.tolist(), "lse": lse.tolist()}, f)
    print("wrote", path)


if __name__ == "__main__":
    main()
