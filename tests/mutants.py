"""Planted mistakes in copies of oracle functions, for checking that a pin bites.

``mutant(fn, old, new)`` returns a copy of the oracle function ``fn`` whose
source has the text ``old`` replaced by ``new`` (which must occur exactly
once; further pairs may follow), compiled against a copy of the oracle
module's globals. The oracle itself is never modified: the copy lives only in
the calling test.
"""
import inspect
import textwrap


def mutant(fn, old: str, new: str, *more: str):
    """``more`` holds further (old, new) pairs, applied in order."""
    src = textwrap.dedent(inspect.getsource(fn))
    pairs = [(old, new)] + list(zip(more[::2], more[1::2]))
    for a, b in pairs:
        n = src.count(a)
        if n != 1:
            raise ValueError(f"{fn.__name__}: {a!r} occurs {n} times, expected once")
        src = src.replace(a, b)
    ns = dict(fn.__globals__)
    exec(compile(src, f"<mutant of {fn.__name__}>", "exec"), ns)
    return ns[fn.__name__]
