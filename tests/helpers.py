"""Small parsing helpers for the golden fixtures in tests/golden/."""
import os
import re

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_PAIR = re.compile(r"\((-?\d+),(-?\d+)\)")


def lines(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for raw in f:
            s = raw.strip()
            if s and not s.startswith("#"):
                yield s


def pairs(text):
    return [(int(a), int(b)) for a, b in _PAIR.findall(text)]


def table(name, prefix):
    """Lines 'prefix <key>: (a,b) (c,d) ...' -> {key: [(a,b), ...]}."""
    out = {}
    for s in lines(name):
        if s.startswith(prefix + " ") and ":" in s:
            head, body = s.split(":", 1)
            key = head[len(prefix):].strip()
            out[key] = pairs(body)
    return out


def keyed(name, key):
    """All lines starting with `key ` -> list of remaining token lists."""
    return [s.split()[1:] for s in lines(name) if s.split()[0] == key]
