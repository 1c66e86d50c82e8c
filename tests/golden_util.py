"""Readers for the cited fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table() -> dict:
    """code -> value, from the OCP MX v1.0 FP4 (E2M1) table fixture."""
    rows = [line.split() for line in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if line.strip() and not line.startswith("#")]
    return {int(c): float(v) for c, v in rows}
