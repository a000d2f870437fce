"""Values the pages print, checked against the oracle (CPU only).

The pages print no worked example of an output or a state; the fixtures under
tests/golden/ hold the numbers they do print that the oracle's pieces can reproduce.
"""

import os

import numpy as np

from oracle import chunk_quantities, inverse_neumann

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def test_stress_power_magnitudes_match_k3_table():
    # R built by the oracle's literal chunk definitions from the stress input; the
    # Neumann product's highest power and largest power entry must match the page.
    for C, hp, mag in _rows("k3_stress_powers.txt"):
        C, hp = int(C), int(hp)
        D = 8
        key = np.ones(D) / np.sqrt(D)
        k = np.tile(key, (C, 1))
        g = np.full((C, D), -0.01)
        beta = np.full(C, 0.5)
        w = chunk_quantities(k, k, g, beta, 1.0)
        _, exponent, max_mag = inverse_neumann(w["R"], return_powers=True)
        assert exponent == hp
        if mag == "inf":
            assert max_mag > float(np.finfo(np.float16).max)
        else:
            # The page accumulated in FP16; FP64 agrees to about 1%.
            assert abs(max_mag - float(mag)) / float(mag) < 0.015, (C, max_mag, mag)


def test_exponent_boundary_counts_match_k3_table():
    tiny = np.finfo(np.float32).tiny
    bf16_max = float(np.float32(3.3895313892515355e38))
    for C, zeros, infs in _rows("k3_exponent_boundary.txt"):
        C = int(C)
        G = np.cumsum(np.full(C, -5.0))
        with np.errstate(over="ignore"):
            up = np.exp2(np.float32(G * np.log2(np.e)))
            down = np.exp2(np.float32(-G * np.log2(np.e)))
        up = np.where(up < tiny, 0.0, up)
        n_zero = int(np.sum(up == 0.0))
        n_inf = int(np.sum(~np.isfinite(down) | (down > bf16_max)))
        assert (n_zero, n_inf) == (int(zeros), int(infs)), C


def test_lower_bound_cliff_is_log_min_normal_over_chunk():
    (chunk, cliff, lb_min), = _rows("fi_lower_bound_cliff.txt")
    derived = np.log(np.finfo(np.float32).tiny) / int(chunk)
    assert abs(derived - float(cliff)) < 1e-4
    # The accepted bound keeps a full 16-token prefix representable in FP32.
    assert np.exp(np.float32(float(lb_min) * int(chunk))) > np.finfo(np.float32).tiny
