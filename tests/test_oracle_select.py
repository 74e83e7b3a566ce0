"""Pins of the transition-cache selection oracle against definitions it does
not use itself: the base argmax when there is no transition, a brute-force
greedy walk over the full score matrix when every token is a candidate, a
planted transition chain, Python's own sort for the candidates, and
relabelling of the vocabulary."""
import numpy as np

from oracle import select as osel


def rand_case(rng, B, G, V, r, scale=1.0):
    z = rng.standard_normal((B, G, V))
    E = rng.standard_normal((V, r)) * scale
    F = rng.standard_normal((V, r)) * scale
    anchor = rng.integers(0, V, B)
    return z, anchor, E, F


def test_candidates_match_a_plain_sort_with_ties():
    rng = np.random.default_rng(1)
    z = rng.integers(-3, 4, 50).astype(np.float64)  # many ties
    want = sorted(range(50), key=lambda i: (-z[i], i))[:16]
    assert list(osel.candidates(z)) == want


def test_no_transition_is_the_base_argmax():
    rng = np.random.default_rng(2)
    z, anchor, E, F = rand_case(rng, 3, 5, 200, 8)
    tok, sc, cand, _ = osel.select_block(z, anchor, np.zeros_like(E), F)
    np.testing.assert_array_equal(tok, np.argmax(z, axis=2))
    np.testing.assert_allclose(sc, np.max(z, axis=2))
    tok2, _, _, _ = osel.select_block(z, anchor, E, np.zeros_like(F))
    np.testing.assert_array_equal(tok2, np.argmax(z, axis=2))


def test_every_token_a_candidate_equals_brute_force_greedy():
    """V = 16: the candidate restriction is void, so the walk is the greedy
    path of s_t(a, b) = z_t(b) + sum_k E[a, k] F[b, k] over all tokens."""
    rng = np.random.default_rng(3)
    B, G, V, r = 2, 6, 16, 4
    z, anchor, E, F = rand_case(rng, B, G, V, r)
    tok, sc, _, _ = osel.select_block(z, anchor, E, F)
    for b in range(B):
        prev = int(anchor[b])
        for t in range(G):
            best, arg = -np.inf, -1
            for cand in range(V):
                s = z[b, t, cand] + sum(E[prev, k] * F[cand, k] for k in range(r))
                if s > best + 1e-12 or (abs(s - best) <= 1e-12 and z[b, t, cand] > z[b, t, arg]):
                    best, arg = s, cand
            assert tok[b, t] == arg
            assert abs(sc[b, t] - best) < 1e-9
            prev = arg


def test_planted_transition_chain_is_followed():
    """A transition offset that only rewards b = next(a) (a permutation)
    outweighs the base logits: the walk follows the chain from the anchor."""
    rng = np.random.default_rng(4)
    V, G = 16, 7
    nxt = rng.permutation(V)
    E = np.eye(V)
    F = np.zeros((V, V))
    F[nxt, np.arange(V)] = 50.0  # E[a] . F[b] = 50 iff b == nxt[a]
    z = rng.standard_normal((1, G, V))
    tok, _, _, _ = osel.select_block(z, np.array([3]), E, F)
    a = 3
    for t in range(G):
        a = nxt[a]
        assert tok[0, t] == a


def test_relabelling_the_vocabulary_relabels_the_tokens():
    rng = np.random.default_rng(5)
    z, anchor, E, F = rand_case(rng, 2, 4, 300, 6)
    tok, sc, _, _ = osel.select_block(z, anchor, E, F)
    perm = rng.permutation(300)          # new label of old token v: perm[v]
    inv = np.argsort(perm)
    z2, E2, F2 = z[:, :, inv], E[inv], F[inv]
    tok2, sc2, _, _ = osel.select_block(z2, perm[anchor], E2, F2)
    np.testing.assert_array_equal(tok2, perm[tok])
    np.testing.assert_allclose(sc2, sc)
