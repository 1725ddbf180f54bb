"""The top-128 mass diagnostic (oracle/topk_mass.py) against closed forms."""
import numpy as np

from oracle import topk_mass as M


def test_uniform_row_keeps_k_over_v():
    z = np.zeros(4096)
    assert abs(M.topk_mass(z, 1.0, 128) - 128 / 4096) < 1e-12


def test_two_levels():
    # 10 tokens at log(9) above 990 others: the top 10 hold 90/(90+990)
    z = np.zeros(1000)
    z[:10] = np.log(9.0)
    assert abs(M.topk_mass(z, 1.0, 10) - 90 / (90 + 990)) < 1e-12
    # temperature 2 halves the gap: weight 3 each
    assert abs(M.topk_mass(z, 2.0, 10) - 30 / (30 + 990)) < 1e-12


def test_masked_tokens_hold_nothing():
    z = np.full(500, -np.inf)
    z[:50] = np.linspace(0, 1, 50)
    assert M.topk_mass(z, 1.0, 128) == 1.0
    assert M.topk_mass(z, 1.0, 50) == 1.0
