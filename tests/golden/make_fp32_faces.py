"""Write ``fp32_faces.json``: fp32 positions next to a cell face or a TSC half-cell
tie, where rounding the quotient (x - origin)/h in fp32 arithmetic lands on
the face (or the tie) while the exact quotient does not.

The expected cell, fraction and TSC centre come from exact rational
arithmetic (``fractions.Fraction``) on the fp32 values of x, origin and h, not
from the oracle or the GPU library: they are what the support rule of
Pennati & Markidis, Sec. 2.3 (j = floor(u), xi = u - j; the TSC stencil is
centred on j when xi < 1/2 and on j + 1 otherwise) gives for the exact value
of each stored fp32 position. Each case also records what fp32 arithmetic
would decide, so a test can show that the cases separate the two readings.

Run from the repository root: python tests/golden/make_fp32_faces.py
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(v) -> np.float32:
    return np.float32(v)


def exact(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def scan(h: float, origin: float, n: int, targets, want: str, limit: int):
    """fp32 positions near origin + t*h for each target t (an integer face, or
    j + 1/2 for the TSC tie) whose fp32 quotient equals t while the exact one
    is below it."""
    hf, of = f32(h), f32(origin)
    H, O = exact(hf), exact(of)
    out = []
    for t in targets:
        x0 = f32(float(of) + float(t) * float(hf))
        for k in range(-6, 7):
            x = x0
            step = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
            for _ in range(abs(k)):
                x = np.nextafter(x, step)
            q32 = (np.float32(x) - of) / hf  # IEEE fp32 subtraction and division
            qx = (exact(x) - O) / H           # exact rational quotient of the stored values
            if Fraction(float(q32)) != Fraction(t) or qx >= Fraction(t):
                continue
            j = math.floor(qx)
            xi = qx - j
            # fp64 arithmetic must agree with the exact decision for the case to be usable
            u64 = (float(x) - float(of)) / float(hf)
            if math.floor(u64) != j:
                continue
            case = {"x": float(x), "x_hex": float(x).hex(), "h": float(hf), "origin": float(of), "n": n,
                    "target": str(t), "exact_quotient": str(qx), "exact_cell": j % n,
                    "exact_xi": str(xi), "exact_xi_float": float(xi),
                    "fp32_quotient": float(q32)}
            if want == "face":
                case["fp32_cell"] = int(math.floor(float(q32))) % n
            else:
                case["exact_tsc_centre"] = (j + (0 if xi < Fraction(1, 2) else 1)) % n
                j32 = math.floor(float(q32))
                xi32 = float(q32) - j32
                case["fp32_tsc_centre"] = (j32 + (0 if xi32 < 0.5 else 1)) % n
            out.append(case)
            if len(out) >= limit:
                return out
    return out


def main():
    n = 8
    faces = scan(0.1, 0.0, n, [Fraction(t) for t in range(1, 8)], "face", 4)
    faces += scan(0.3, -0.7, n, [Fraction(t) for t in range(1, 8)], "face", 3)
    ties = scan(0.1, 0.0, n, [Fraction(2 * t + 1, 2) for t in range(0, 8)], "tie", 4)
    ties += scan(0.3, -0.7, n, [Fraction(2 * t + 1, 2) for t in range(0, 8)], "tie", 3)
    doc = {
        "source": "Pennati & Markidis, Mass Matrix Assembly on Tensor Cores for Implicit Particle-In-Cell "
                  "Methods, Sec. 2.3 (support rule: j = floor(u), xi = u - j, TSC centred on j if xi < 1/2 else "
                  "j + 1) and Sec. 5 (fp32 storage of positions).",
        "note": "fp32 positions whose fp32-arithmetic quotient (x - origin)/h lands exactly on a face (faces) or on "
                "a TSC half-cell tie (ties) while the exact quotient of the stored values is just below it. "
                "Expected values are exact rational arithmetic on the stored fp32 values (this script); the "
                "fp32_* fields record the other reading, which these cases must contradict.",
        "faces": faces,
        "ties": ties,
    }
    with open(os.path.join(HERE, "fp32_faces.json"), "w") as f:
        json.dump(doc, f, indent=1)
    print(f"{len(faces)} face cases, {len(ties)} tie cases")


if __name__ == "__main__":
    main()
