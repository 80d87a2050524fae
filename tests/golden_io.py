"""Parser for the worked-example fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    rec = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            rec.setdefault(key, []).append(vals)
    return rec


def scalar(rec, key, cast=int):
    return cast(rec[key][0][0])
