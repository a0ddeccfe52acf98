"""Reader for the `key: values` golden fixture files under tests/golden/."""
import os
from typing import Dict, List

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_kv(name: str) -> Dict[str, List[str]]:
    out: Dict[str, List[str]] = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line or ":" not in line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


def read_lines(name: str) -> List[str]:
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split("#", 1)[0].strip() for ln in f if ln.split("#", 1)[0].strip()]


def hexu32(vals: List[str]) -> List[int]:
    return [int(v, 16) for v in vals]
