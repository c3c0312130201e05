"""Readers for the hand-worked fixtures under tests/golden/."""
import math
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def closed_form(expr: str) -> float:
    """Evaluate a hand-written closed form such as 'exp(2)/(exp(2)+1)'."""
    env = {"exp": math.exp, "e": math.e, "nan": float("nan"), "__builtins__": {}}
    return float(eval(expr, env))


def kv(name):
    out = {}
    for ln in lines(name):
        key, *vals = ln.split()
        out[key] = vals
    return out
