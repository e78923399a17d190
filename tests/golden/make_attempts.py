"""Write tests/golden/attempts.json: per workload, the first draft attempt of each
sequence that passes the near-tie rule (computed with the oracle only).

    python tests/golden/make_attempts.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from ddt_synthetic import configs  # noqa: E402
from _cases import ATTEMPTS_FILE, pick_attempt  # noqa: E402


def main():
    table = {}
    for name in ["C0", "C1", "C2", "C3", "C4"]:
        cfg = configs.C3[512] if name == "C3" else configs.get(name)
        S = 64 if name == "C0" else cfg.S   # extra tiny draws for multi-seed tests
        table[name] = [pick_attempt(cfg, s) for s in range(S)]
        print(name, table[name], flush=True)
    with open(ATTEMPTS_FILE, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
