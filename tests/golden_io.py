"""Reader for the text fixtures under tests/golden/ (blocks of numbers)."""

import os
import re

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_blocks(name):
    """{block name: (array, tolerance or None)} from a fixture file."""
    blocks = {}
    cur, tol, rows = None, None, []

    def flush():
        if cur is not None:
            blocks[cur] = (np.array(rows, dtype=np.float64), tol)

    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            m = re.match(r"^\[(\w+)(?:\s+tol=([0-9.eE+-]+))?\]$", line)
            if m:
                flush()
                cur, tol, rows = m.group(1), (float(m.group(2)) if m.group(2) else None), []
            else:
                rows.append([float(t) for t in line.split()])
    flush()
    return {k: ((v[0][0] if v[0].shape[0] == 1 else v[0]), v[1]) for k, v in blocks.items()}


def worked_example():
    """Q, K, V of the worked example and the printed expectations."""
    b = load_blocks("worked_example_n8_d4_b4.txt")
    Q, K = b.pop("Q")[0], b.pop("K")[0]
    V = np.eye(8)[:, :4]
    return Q, K, V, b
