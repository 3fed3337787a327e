"""Shared pytest setup: the ``gpu`` marker and small helpers.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; the
rest run on any host.
"""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def load_golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def golden_q2k_block(spec):
    """Assemble an 84-byte Q2K block from a golden entry's fields."""
    def expand(lst, n):
        out = []
        i = 0
        while i < len(lst):
            v = int(lst[i], 16)
            if i + 1 < len(lst) and isinstance(lst[i + 1], int):
                out += [v] * lst[i + 1]
                i += 2
            else:
                out.append(v)
                i += 1
        assert len(out) == n, (spec["id"], len(out))
        return out
    scales = expand(spec["scales"], 16)
    head = [int(h, 16) for h in spec["codes_head"]]
    codes = head + [int(spec["codes_fill"], 16)] * (64 - len(head))
    d = int(spec["d"], 16)
    dm = int(spec["dmin"], 16)
    return bytes(scales + codes + [d & 0xFF, d >> 8, dm & 0xFF, dm >> 8])
