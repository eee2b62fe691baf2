"""Reader of the text fixtures in this folder: `key: value` lines, `#` comments (citations) skipped."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, value = line.partition(":")
            out[key.strip()] = value.strip()
    return out


def hex_bytes(value):
    return bytes(int(t, 16) for t in value.split())
