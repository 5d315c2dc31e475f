"""Reader for the small text fixtures under tests/golden/ (key value... lines,
'#' comments carry the citation)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def num(vals):
    def conv(v):
        return int(v, 16) if v.startswith("0x") else float(v)
    return [conv(v) for v in vals] if len(vals) > 1 else conv(vals[0])
