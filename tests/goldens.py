"""Readers for the hand-worked fixtures in tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def f32(hexbits):
    return np.array([int(hexbits, 16)], dtype=np.uint32).view(np.float32)[0]


def e4m3_cases():
    """[(fp32 value, expected code)]"""
    out = []
    for line in _lines("e4m3_encode_cases.txt"):
        bits, code = line.split()[:2]
        out.append((f32(bits), int(code, 16)))
    return out


def quant_tile_cases():
    """[(name, tile float32[128], scale float32, codes uint8[128])]"""
    cases, cur = [], None
    for line in _lines("quant_tile_cases.txt"):
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = {"name": rest.strip(), "tile": np.zeros(128, np.float32),
                   "codes": np.zeros(128, np.uint8)}
        elif key == "tile":
            for kv in rest.split():
                i, v = kv.split(":")
                cur["tile"][int(i)] = f32(v)
        elif key == "scale":
            cur["scale"] = f32(rest.strip())
        elif key == "codes":
            for kv in rest.split():
                i, v = kv.split(":")
                cur["codes"][int(i)] = int(v, 16)
        elif key == "end":
            cases.append((cur["name"], cur["tile"], cur["scale"], cur["codes"]))
            cur = None
    return cases


def gemm_hand_case():
    """Inputs of the hand-worked GEMM case and its expected outputs.

    Returns (a float32 [1][128], b float32 [128][128], expected dict) where
    expected[('fp32'|'bf16', 'n0'|'n_other')] is the value of C[0][0] / C[0][n>=1].
    """
    a = np.ones((1, 128), np.float32)
    a[0, 0] = 448.0
    b = np.full((128, 128), 0.5, np.float32)
    b[0, 0] = 448.0
    exp = {}
    for line in _lines("gemm_hand_cases.txt"):
        kind, which, val = line.split()
        exp[(kind, which)] = float(val)
    return a, b, exp
