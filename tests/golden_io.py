"""Readers for the text fixtures under tests/golden/."""

from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand(tokens):
    vals = []
    for tok in tokens:
        if "*" in tok:
            v, n = tok.split("*")
            vals.extend([int(v, 16)] * int(n))
        else:
            vals.append(int(tok, 16))
    return vals


def read_worked_example(name: str) -> dict:
    """`key: hex hex ...` lines (HEX*n repeats a value); R, T, H are decimal; `scale` is kept as text."""
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(":")
            key, rest = key.strip(), rest.strip()
            if key in ("R", "T", "H"):
                d[key] = int(rest)
            elif key == "scale":
                d[key] = rest
            else:
                d[key] = _expand(rest.split())
    T, H = d["T"], d["H"]
    out = {"R": d["R"], "T": T, "H": H}
    out["partials"] = np.array([d[f"P{r}"] for r in range(d["R"])], dtype=np.uint16).reshape(d["R"], T, H)
    out["residual"] = np.array(d["residual"], np.uint16).reshape(T, H) if "residual" in d else None
    out["gamma"] = np.array(d["gamma"], np.uint16)
    for k in ("residual_out", "out"):
        out[k] = np.array(d[k], np.uint16).reshape(T, H)
    if "q" in d:
        out["q"] = np.array(d["q"], np.uint8).reshape(T, H)
    if "scale" in d:
        out["scale"] = d["scale"]
    return out


def read_value_code_table(name: str):
    """Lines `<python float expression> <hex code>`; returns [(value, code)]."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            expr, code = line.rsplit(None, 1)
            rows.append((float(eval(expr, {"__builtins__": {}}, {})), int(code, 16)))
    return rows
