"""Loader of the small text fixtures in this folder (values printed on the pages)."""
import os

_HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    """Parse 'key: v v v' lines; ints where possible.  '#' lines are comments."""
    out = {}
    with open(os.path.join(_HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            vals = v.split()
            try:
                out[k.strip()] = [int(x) for x in vals]
            except ValueError:
                out[k.strip()] = vals
    return out
