"""Readers of the golden fixtures (see README.md in this folder)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def rows(name):
    """The non-comment lines of a fixture, split into fields."""
    out = []
    with open(os.path.join(HERE, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out
