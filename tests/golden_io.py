"""Reader for the golden fixture files under tests/golden/."""
from __future__ import annotations

import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    """Parse one fixture: returns causal, scale, q, k, v (float64 2-D), and
    weights/out as (matrix, tolerance)."""
    out: dict = {}
    key = None
    rows: list = []

    def flush():
        if key is None:
            return
        mat = np.array(rows, dtype=np.float64)
        if isinstance(out.get(key), float):
            out[key] = (mat, out[key])
        else:
            out[key] = mat

    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] in ("causal", "scale"):
                flush()
                key = None
                out[tok[0]] = int(tok[1]) if tok[0] == "causal" else float(tok[1])
            elif tok[0] in ("q", "k", "v", "weights", "out"):
                flush()
                key, rows = tok[0], []
                if len(tok) > 1:
                    out[key] = float(tok[1])
            else:
                rows.append([float(t) for t in tok])
    flush()
    return out
