"""The spherical binning kernel's angle estimate: its polynomial constants
are what the comment in spherical.hip says they are (a least-squares fit of
atan(t)/t in powers of t^2 on [0, 1], degree 6), and the estimate evaluated
in float32 as the kernel does stays within the error it states (7e-7 rad).
The estimate only seeds exact boundary tests, so this pins the constants'
provenance, not any output."""
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "sparse_spatial_hashing_amd", "csrc", "spherical.hip")


def kernel_coefficients():
    text = open(SRC).read()
    body = text[text.index("float atan2_estimate("):]
    body = body[:body.index("\n}\n")]
    lead = re.search(r"float q = ([0-9.e+-]+)f;", body)
    steps = re.findall(r"q = q \* u ([+-]) ([0-9.e+-]+)f;", body)
    # Horner from the highest power: q = c6; q = q u + c5; ... ; q = q u + c0
    coef = [float(lead.group(1))] + [float(v) * (1 if s == "+" else -1) for s, v in steps]
    return np.array(coef[::-1])  # c0 .. c6


def test_constants_are_the_least_squares_fit():
    c = kernel_coefficients()
    assert c.shape == (7,)
    t = np.linspace(0.0, 1.0, 200001)[1:]
    V = np.vander(t * t, 7, increasing=True)
    fit = np.linalg.lstsq(V, np.arctan(t) / t, rcond=None)[0]
    assert np.max(np.abs(fit - c)) < 1e-3, (fit, c)


def test_float32_estimate_within_stated_error():
    c = kernel_coefficients().astype(np.float32)
    t = np.linspace(0.0, 1.0, 400001, dtype=np.float64).astype(np.float32)
    u = (t * t).astype(np.float32)
    q = np.full_like(u, c[6])
    for k in range(5, -1, -1):
        q = (q * u).astype(np.float32) + c[k]
        q = q.astype(np.float32)
    r = (t * q).astype(np.float32)
    err = np.abs(r.astype(np.float64) - np.arctan(t.astype(np.float64)))
    assert err.max() < 7e-7, err.max()
