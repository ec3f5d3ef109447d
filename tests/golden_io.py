"""Readers for the hand-worked fixtures in tests/golden/ (plain text, '#' comments)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            s = raw.strip()
            if s and not s.startswith("#"):
                yield s


def matrices(name):
    """Blocks 'NAME rows cols' followed by rows of numbers."""
    out = {}
    it = iter(lines(name))
    for head in it:
        key, r, c = head.split()
        r, c = int(r), int(c)
        out[key] = np.array([[float(v) for v in next(it).split()] for _ in range(r)], dtype=np.float64)
        assert out[key].shape == (r, c)
    return out


def projection_cases():
    return [tuple(float(v) for v in s.split()[:2]) + (int(s.split()[2]),) for s in lines("projection_cases.txt")]


def quantize_hand():
    d = {"codes": {}, "scales": {}, "normsq": {}}
    for s in lines("quantize_hand.txt"):
        f = s.split()
        if f[0] in ("U_re", "U_im", "W_re", "W_im"):
            d[f[0]] = np.array([float(v) for v in f[1:]])
        elif f[0] == "codes":
            d["codes"][(f[1], int(f[2]))] = [int(v) for v in f[3:]]
        elif f[0] == "scales":
            d["scales"][(f[1], int(f[2]))] = (float(f[3]), float(f[4]))
        elif f[0] == "normsq":
            d["normsq"][f[1]] = [float(v) for v in f[2:]]
    return d


def pack_bytes():
    return [tuple(int(v) for v in s.split()) for s in lines("pack_bytes.txt")]


def pack_tile_order():
    """-> (total bytes, [(t, M, i, j, byte offset, bit shift)]) for n = 20, m = 320, T = 2."""
    total, rows = None, []
    for s in lines("pack_tile_order.txt"):
        f = s.split()
        if f[0] == "total":
            total = int(f[1])
        else:
            rows.append(tuple(int(v) for v in f))
    return total, rows


def storage_bits():
    return [tuple(int(v) for v in s.split()) for s in lines("storage_bits.txt")]


def gemv_hand():
    d = {"codes": {}, "scales": {}, "y": {}}
    for s in lines("gemv_hand.txt"):
        f = s.split()
        if f[0] == "x":
            d["x"] = np.array([float(v) for v in f[1:]])
        elif f[0] == "codes":
            d["codes"][(f[1], int(f[2]))] = [int(v) for v in f[3:]]
        elif f[0] == "scales":
            d["scales"][(f[1], int(f[2]))] = (float(f[3]), float(f[4]))
        elif f[0] == "y":
            d["y"][f[1]] = np.array([float(v) for v in f[2:]])
    return d


def act_quant_hand():
    toks = []
    cur = {}
    for s in lines("act_quant_hand.txt"):
        f = s.split()
        if f[0] == "x":
            cur = {"x": np.array([float(v) for v in f[1:]])}
        elif f[0] == "q":
            cur["q"] = np.array([int(v) for v in f[1:]])
        elif f[0] == "delta":
            cur["delta"] = float(f[1])
            toks.append(cur)
    return toks


def order_sum_cases():
    out = []
    for s in lines("order_sum.txt"):
        left, right = s.split("->")
        f = left.split()
        m = int(f[0])
        entries = {int(a): float(b) for a, b in (e.split(":") for e in f[1:])}
        out.append((m, entries, float(right)))
    return out


def tensor_order_cases():
    """-> [(n, {row: Re U value}, expected per-tensor s_re)] from tensor_order.txt."""
    out = []
    for s in lines("tensor_order.txt"):
        left, right = s.split("->")
        f = left.split()
        rows = {int(a): float(int(b)) for a, b in (e.split(":") for e in f[1:])}
        out.append((int(f[0]), rows, float(int(right))))
    return out
