"""Pins for the oracle's offline high-risk row selection (CPU only).

The score is mean row energy times the retention factor 1/(1 - abar) of a gate that scales the
state by abar per step (DAMP abstract: quantization error together with decay-based error
retention). Pinned by a planted closed form (rows of constant value, known energies and gates),
by tie-breaking to the lower index, and by a brute-force Python ranking on random states.
"""
import numpy as np

import oracle


def test_planted_energies_and_gates():
    D, H = 16, 2
    e = np.linspace(0.5, 2.0, D)          # row energies (mean square)
    abar = np.zeros((H, D))
    abar[0] = 0.5                          # head 0: equal gates -> ranking by energy alone
    abar[1] = np.linspace(0.0, 0.9, D)[::-1]   # head 1: slow gates on low-energy rows
    S = np.empty((3, H, D, D), np.float32)
    for i in range(D):
        S[:, :, i, :] = np.float32(np.sqrt(e[i]))
    rows, score = oracle.select_rows(S, abar, 4)
    want_score = np.stack([np.float32(np.sqrt(e)).astype(np.float64) ** 2 / (1 - abar[h])
                           for h in range(H)])
    np.testing.assert_allclose(score, want_score, rtol=1e-12)
    assert rows[0].tolist() == [12, 13, 14, 15]
    closed = e / (1 - abar[1])
    assert rows[1].tolist() == sorted(np.argsort(-closed, kind="stable")[:4].tolist())
    assert rows[1].tolist() != rows[0].tolist()   # the decay term changes the choice


def test_ties_go_to_lower_index():
    D, H = 8, 1
    S = np.ones((2, H, D, D), np.float32)
    rows, _ = oracle.select_rows(S, np.full((H, D), 0.3), 3)
    assert rows.tolist() == [[0, 1, 2]]


def test_random_against_bruteforce_ranking():
    rng = np.random.default_rng(31)
    n, H, D, r = 5, 3, 32, 6
    S = (rng.standard_normal((n, H, D, D)) * rng.lognormal(0, 1, (1, H, D, 1))).astype(np.float32)
    abar = rng.uniform(0, 0.99, (H, D))
    rows, score = oracle.select_rows(S, abar, r)
    for h in range(H):
        sc = [np.mean([np.mean(S[s, h, i].astype(np.float64) ** 2) for s in range(n)])
              / (1 - abar[h, i]) for i in range(D)]
        np.testing.assert_allclose(score[h], sc, rtol=1e-12)
        best = sorted(range(D), key=lambda i: (-sc[i], i))[:r]
        assert rows[h].tolist() == sorted(best)
