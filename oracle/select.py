"""Oracle of block token selection through a transition cache (test
infrastructure only).

DSpine article, "principle": each block position first keeps its 16 best
candidate tokens; the scores of every pairing of a candidate at one position
with a candidate at the next are computed at once into a 16 x 16 table (the
transition cache); tokens are then chosen from left to right by looking up
the table row of the token just chosen, with no further matrix work per step.
The message from the predecessor enters through a fixed low-dimensional token
representation table (same section).  DSpark tutorial, "semi-autoregressive
generation": the Markov head adds to each position's logits an offset that
depends only on the immediately preceding token, through a low-rank (rank
256) factorisation of the transition matrix.

Readings taken where the pages leave a step open:
  * The score of token b at drafted position t after token a is
    s_t(a, b) = z_t(b) + E[a] . F[b]: the position's base logit plus the
    rank-r transition offset, E [V, r] being the predecessor's representation
    and F [V, r] the successor's (bf16 tables; products summed in float64
    here).
  * Candidates of position t: the 16 largest z_t (value desc, index asc).
  * Position 0's predecessor is the anchor (the round's last committed token),
    so its row of the table is s_0(anchor, c_0[j]); position t >= 1 uses the
    candidates of t - 1 as rows: T_t[i][j] = s_t(c_{t-1}[i], c_t[j]).
  * Selection: j_0 = argmax_j T_0[j], j_t = argmax_j T_t[j_{t-1}][j], ties to
    the lower j (the better base logit); the drafted tokens are c_t[j_t].
"""
import numpy as np

N_CAND = 16


def candidates(z: np.ndarray, n: int = N_CAND) -> np.ndarray:
    """Indices of the n largest entries of z, value descending, index
    ascending among equal values."""
    z = np.asarray(z, dtype=np.float64)
    order = np.lexsort((np.arange(z.shape[0]), -z))
    return order[:min(n, z.shape[0])]


def transition_table(z: np.ndarray, E: np.ndarray, F: np.ndarray, prev: np.ndarray, cand: np.ndarray) -> np.ndarray:
    """T[i][j] = z[cand[j]] + E[prev[i]] . F[cand[j]] for predecessor tokens
    prev and candidate tokens cand of one position."""
    E = np.asarray(E, dtype=np.float64)
    F = np.asarray(F, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    return z[cand][None, :] + E[prev] @ F[cand].T


def select_block(z: np.ndarray, anchor: np.ndarray, E: np.ndarray, F: np.ndarray):
    """z [B, G, V] base logits of the drafted positions, anchor [B] int,
    E, F [V, r].  Returns (tokens [B, G] int32, scores [B, G] float64 (the
    chosen table entries), cand [B, G, 16] int32, tables [B, G, 16, 16]
    float64 (row 0 only for position 0))."""
    z = np.asarray(z)
    B, G, V = z.shape
    n = min(N_CAND, V)
    tokens = np.zeros((B, G), np.int32)
    scores = np.zeros((B, G))
    cand = np.zeros((B, G, n), np.int32)
    tables = np.zeros((B, G, n, n))
    for b in range(B):
        for t in range(G):
            cand[b, t] = candidates(z[b, t], n)
        j_prev = -1
        for t in range(G):
            prev = np.array([anchor[b]]) if t == 0 else cand[b, t - 1]
            T = transition_table(z[b, t], E, F, prev, cand[b, t])
            tables[b, t, :T.shape[0]] = T
            row = T[0] if t == 0 else T[j_prev]
            j = int(np.argmax(row))  # first maximum: the lower j on ties
            tokens[b, t] = cand[b, t, j]
            scores[b, t] = row[j]
            j_prev = j
    return tokens, scores, cand, tables
