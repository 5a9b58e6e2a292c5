"""Small helpers shared by the tests (no convolution arithmetic here)."""

import ast
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def eval_expr(text):
    """Evaluate a fixture expression: numbers, + - * / ** and sqrt() only."""
    node = ast.parse(str(text), mode="eval").body

    def ev(n):
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, (ast.USub, ast.UAdd)):
            v = ev(n.operand)
            return -v if isinstance(n.op, ast.USub) else v
        if isinstance(n, ast.BinOp):
            a, b = ev(n.left), ev(n.right)
            if isinstance(n.op, ast.Add):
                return a + b
            if isinstance(n.op, ast.Sub):
                return a - b
            if isinstance(n.op, ast.Mult):
                return a * b
            if isinstance(n.op, ast.Div):
                return a / b
            if isinstance(n.op, ast.Pow):
                return a ** b
        if (isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id == "sqrt"
                and len(n.args) == 1):
            return math.sqrt(ev(n.args[0]))
        raise ValueError(f"unsupported expression {text!r}")

    return ev(node)


def eval_array(nested):
    if isinstance(nested, list):
        return np.array([eval_array(v) for v in nested], dtype=np.float64)
    return eval_expr(nested)


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def random_rotation(rng):
    axis = rng.standard_normal(3)
    angle = rng.uniform(0.1, math.pi)
    return axis / np.linalg.norm(axis), angle


def rel_max_err(a, ref):
    ref = np.asarray(ref, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(np.asarray(a, dtype=np.float64) - ref))) if ref.size else 0.0
    return err / rms if rms > 0 else err
