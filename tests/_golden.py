"""Reader for the small hand-worked fixtures under ``tests/golden/``.

Format: ``#`` starts a comment; a line with one word opens a block whose
following numeric lines form a 2D array; ``key value`` sets a scalar.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out: dict = {}
    key = None
    rows: list = []

    def flush():
        if key is not None and rows:
            out[key] = np.array(rows, dtype=np.int64)

    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            try:
                nums = [int(p) for p in parts]
            except ValueError:
                nums = None
            if nums is not None:
                rows.append(nums)
                continue
            flush()
            rows = []
            if len(parts) == 2:
                out[parts[0]] = int(parts[1])
                key = None
            else:
                key = parts[0]
    flush()
    return out
