"""Exact evaluation of the hand-worked closed forms in ``tests/golden``.

An expression is a string over decimal literals, ``+ - * / **``, parentheses,
the functions ``sqrt``, ``exp`` and ``ln`` and the name ``eps``.  It is parsed
with :mod:`ast` (never ``eval``) and evaluated in :mod:`decimal` arithmetic at
50 significant digits, then rounded once, to nearest with ties to even, to
float32 or float16.
"""
from __future__ import annotations

import ast
import decimal
from decimal import Decimal

import numpy as np

_CTX = decimal.Context(prec=50)


def evaluate(expr: str, eps: Decimal = Decimal(0)) -> Decimal:
    tree = ast.parse(expr, mode="eval")

    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            # Use the literal's text so that 0.1 means one tenth exactly.
            return Decimal(ast.get_source_segment(expr, node))
        if isinstance(node, ast.Name) and node.id == "eps":
            return eps
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, (ast.USub, ast.UAdd)):
            v = ev(node.operand)
            return _CTX.minus(v) if isinstance(node.op, ast.USub) else v
        if isinstance(node, ast.BinOp):
            a, b = ev(node.left), ev(node.right)
            if isinstance(node.op, ast.Add):
                return _CTX.add(a, b)
            if isinstance(node.op, ast.Sub):
                return _CTX.subtract(a, b)
            if isinstance(node.op, ast.Mult):
                return _CTX.multiply(a, b)
            if isinstance(node.op, ast.Div):
                return _CTX.divide(a, b)
            if isinstance(node.op, ast.Pow):
                return _CTX.power(a, b)
        if isinstance(node, ast.Call) and isinstance(node.func, ast.Name) and len(node.args) == 1:
            v = ev(node.args[0])
            if node.func.id == "sqrt":
                return _CTX.sqrt(v)
            if node.func.id == "exp":
                return _CTX.exp(v)
            if node.func.id == "ln":
                return _CTX.ln(v)
        raise ValueError(f"unsupported construct in closed form {expr!r}: {ast.dump(node)}")

    return ev(tree)


def round_to(value: Decimal, dtype) -> np.generic:
    """The dtype value nearest to ``value`` (ties to the even significand)."""
    dtype = np.dtype(dtype)
    first = dtype.type(float(value))
    if not np.isfinite(first):
        return first
    cands = [np.nextafter(first, dtype.type(-np.inf)), first,
             np.nextafter(first, dtype.type(np.inf))]
    uint = np.uint16 if dtype.itemsize == 2 else np.uint32

    def key(c):
        err = abs(Decimal(float(c)) - value)
        odd = int(np.array(c, dtype).view(uint)) & 1
        return (err, odd)

    return min(cands, key=key)
