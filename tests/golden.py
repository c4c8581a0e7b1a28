"""Reader of the text fixtures in tests/golden (key value... lines, '#' comments)."""
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        for line in f:
            line = line.rstrip("\n")
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if rest.startswith("|") and rest.endswith("|"):
                out[key] = rest[1:-1]
            else:
                vals = rest.split()
                out[key] = [int(v) for v in vals] if all(v.lstrip("-").isdigit() for v in vals) else vals
    return out
