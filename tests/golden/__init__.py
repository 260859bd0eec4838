"""Loader for the hand-derived text fixtures in this folder."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    """Parse 'key: values' lines (comments start with '#') into a dict of
    lists of floats; keys that repeat with an index ('row 3') become dicts."""
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            vals = [float(x) for x in val.split()]
            parts = key.split()
            if len(parts) == 2:
                out.setdefault(parts[0], {})[int(parts[1])] = vals
            else:
                out[key] = vals
    return out
