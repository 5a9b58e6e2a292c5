"""Irreps strings for the oracle (test infrastructure; see ``oracle/__init__``).

An irreps string lists blocks ``MULxLP`` joined by ``+``, for example
``"8x0e + 8x1o"`` (8 copies of l=0 even, 8 copies of l=1 odd).  This follows
the e3nn-style strings shown on the e3nn_mlx gate-points page (Public API) and
the irreps used by the cuEquivariance skill page (layouts section).  A
multiplicity may distribute over a parenthesised group, ``"64x(0e+1o+2e)"``
meaning ``"64x0e+64x1o+64x2e"``.  A block with no ``MULx`` has multiplicity 1.

Component order (the e3j ``Convolution.__call__`` shapes with trailing
channels): blocks in the order listed, then ``m = -l..l`` inside a block; the
multiplicity is the trailing channel axis, so a uniform multiplicity ``C`` is
required by the convolution.
"""

import re

_BLOCK = re.compile(r"^(?:(\d+)\s*x\s*)?(\d+)\s*([eo])$")


def _split_top(s):
    parts, depth, cur = [], 0, ""
    for ch in s:
        if ch == "(":
            depth += 1
        elif ch == ")":
            depth -= 1
            if depth < 0:
                raise ValueError("unbalanced parentheses in irreps string")
        if ch == "+" and depth == 0:
            parts.append(cur)
            cur = ""
        else:
            cur += ch
    if depth != 0:
        raise ValueError("unbalanced parentheses in irreps string")
    parts.append(cur)
    return [p.strip() for p in parts]


def parse(s):
    """Return a list of ``(mul, l, parity)`` with parity +1 ('e') or -1 ('o')."""
    if not isinstance(s, str) or not s.strip():
        raise ValueError("empty irreps string")
    out = []
    for part in _split_top(s.replace(" ", "")):
        if not part:
            raise ValueError(f"empty block in irreps string {s!r}")
        group = re.match(r"^(\d+)x\((.*)\)$", part)
        if group:
            mul = int(group.group(1))
            for (m2, l, p) in parse(group.group(2)):
                out.append((mul * m2, l, p))
            continue
        m = _BLOCK.match(part)
        if not m:
            raise ValueError(f"bad irreps block {part!r}")
        mul = int(m.group(1)) if m.group(1) is not None else 1
        out.append((mul, int(m.group(2)), 1 if m.group(3) == "e" else -1))
    return out

