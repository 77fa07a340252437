"""Parse the symbolic numbers of the golden fixtures ('ln3', '18/7', '-0', '1+1e-12')."""
import json
import math
import os

import numpy as np

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(HERE, name)) as f:
        return json.load(f)


def num(v):
    if isinstance(v, (int, float)):
        return float(v)
    s = str(v).strip()
    if s == "-0":
        return -0.0
    if s.startswith("ln"):
        return math.log(float(s[2:]))
    if "/" in s:
        a, b = s.split("/")
        return float(a) / float(b)
    if "+" in s[1:]:
        a, b = s.split("+", 1)
        return float(a) + float(b)
    return float(s)


def arr(v):
    if isinstance(v, list):
        if len(v) == 0:
            return np.zeros(0)
        if isinstance(v[0], list):
            return np.array([[num(x) for x in row] for row in v], dtype=np.float64)
        return np.array([num(x) for x in v], dtype=np.float64)
    return np.float64(num(v))
