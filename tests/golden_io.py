"""Readers for the hand-worked fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(expr: str) -> float:
    # fixtures hold plain numeric expressions such as 3*2**-10
    return float(eval(expr, {"__builtins__": {}}, {}))


def e4m3_hand_values():
    out = []
    with open(os.path.join(GOLDEN, "e4m3_hand_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            out.append((_num(parts[0]), int(parts[1], 16)))
    return out


def cast_hand_groups():
    groups, cur = {}, None
    with open(os.path.join(GOLDEN, "cast_hand_groups.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                groups[cur] = {}
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            if key == "fmt":
                groups[cur][key] = val
            elif key == "values":
                groups[cur][key] = [_num(v) for v in val.split(",")]
            elif key == "codes":
                groups[cur][key] = [int(v, 16) for v in val.split(",")]
            else:
                groups[cur][key] = int(val, 0)
    return groups
