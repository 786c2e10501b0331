"""Write tests/golden/descriptor_hashes.json from the CPU oracle only.

For each full-size workload the oracle builds the whole Execution Descriptor
(oracle/descriptor.py) from the seeded metadata (workloads/) and this script
records its SHA-256, so that the GPU test can compare the HIP descriptor
bit-exactly without rebuilding the 32K oracle tables (about 30 s each).

Table widths are the slot counts the workloads' rules need (one interval per
disjunct that cannot be merged over its whole Region):
  causal         rows 1 ([0,i+1))            columns 1 ([j,N))
  shared_prompt  rows 2 ([0,P), [s(i),i+1))  columns 1
  hstu           rows 2 ([0,h), [i,i+1))     columns 1
  retrieval      rows 4 (prefix, own segment, two references)
                 columns 1 + seg_cap (own segment tail, one per segment that
                 may reference it)

    python tests/golden/make_descriptor_hashes.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import descriptor as od  # noqa: E402
from workloads import WORKLOADS, make_metadata  # noqa: E402


def widths(w):
    return {"causal": (1, 1), "shared_prompt": (2, 1), "hstu": (2, 1),
            "retrieval": (4, 1 + w.seg_cap)}[w.mask]


def main():
    out = {}
    for name, w in WORKLOADS.items():
        md = make_metadata(w)
        K_r, K_c = widths(w)
        words = od.build(w.mask, md, K_r, K_c, w.tiles)
        out[name] = {"sha256": hashlib.sha256(words.tobytes()).hexdigest(), "bytes": int(words.nbytes),
                     "K_r": K_r, "K_c": K_c, "tiles": list(w.tiles), "seed": w.seed}
        print(name, out[name], flush=True)
    with open(os.path.join(HERE, "descriptor_hashes.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
