"""Writes synth_sha256.json: the SHA-256 of every input the seeded generator
(synth/) produces for each workload.  Calls only the generator.

    python tests/golden/write_synth_sha256.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402


def main():
    out = {}
    for name in sorted(synth.WORKLOADS):
        w = synth.workload(name)
        out[name] = {k: hashlib.sha256(v.tobytes()).hexdigest() for k, v in sorted(w.inputs().items())}
        print(name, {k: v[:12] for k, v in out[name].items()}, flush=True)
    with open(os.path.join(HERE, "synth_sha256.json"), "w") as f:
        json.dump({"what": "SHA-256 of each generated input (raw bytes: bf16 bits, int64 segment bounds), "
                           "written by write_synth_sha256.py", "workloads": out}, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
