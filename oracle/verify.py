"""Oracle of block verification (test infrastructure only).

DSpark tutorial, "speculative decoding basics": the target scores the whole
drafted block in one pass; drafted tokens are checked from the first one on,
each kept while the target agrees; at the first disagreement a replacement
token is drawn and everything after it is dropped; one more target token is
produced to start the next round.  The same page (and its FAQ) states that the
rejection rule leaves the output distribution equal to the target's; the
standard rule behind this (Leviathan et al., cited by the DFlash/Spec V2 blog
in its reference table) accepts a drafted token d with probability
min(1, P(d)/Q(d)) and otherwise samples from the normalised max(0, P - Q).
DSpine article, "principle": with greedy decoding a drafted token is kept only
while it equals the target's own choice.

Readings taken where the pages leave a step open:
  * K counts the anchor: G = K - 1 drafted tokens d_1..d_G, target logits at
    G + 1 positions, draft logits at G positions; tau counts accepted drafted
    tokens (0..G); each round emits tau + 1 tokens.
  * Greedy (temperature 0): the target's choice is the lowest-index maximum of
    its raw logits; the extra token is that choice at position tau + 1.
  * Sampling: P = filt(softmax(z_t / T)), Q = filt(softmax(z_d / T)) with
    filt = top-k by raw logit (value desc, index asc), softmax over the kept
    set, then top-p: the shortest prefix in (probability desc, index asc)
    order whose sum reaches p (at least one token), renormalised.
  * Accept d_i iff u_i < r_i, r_i = fp32(P_i(d_i)) / fp32(Q_i(d_i)) as an IEEE
    fp32 division (so Q = 0 accepts iff P > 0).
  * Replacement at the first rejection i: weights R = max(0, P_i - Q_i),
    Z = sum R; the token is the smallest x (vocab order) with
    cumsum(R)[x] > u'_i * Z; if rounding leaves none, the last x with R > 0;
    if Z == 0, the weights are P_i.  With every draft accepted, the same draw
    over P_{G+1} with u'_{G+1}.
  * Uniforms [B, G+1, 2]: [b, i, 0] accepts drafted position i, [b, i, 1]
    draws the replacement / extra token at position i.
All probabilities are float64.
"""
import numpy as np

NEAR_TIE = 1e-6


def row_order(z: np.ndarray) -> np.ndarray:
    """Indices of z sorted by value descending, index ascending."""
    idx = np.arange(len(z))
    return np.lexsort((idx, -np.asarray(z, dtype=np.float64)))


def softmax(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def filtered_probs(z: np.ndarray, temperature: float, top_k: int = 0, top_p: float = 1.0) -> np.ndarray:
    """Full-vocabulary probability vector of one row of logits after
    temperature, top-k, softmax over the kept set, and top-p."""
    z = np.asarray(z)
    V = z.shape[0]
    x = z.astype(np.float64) / float(temperature)
    if 0 < top_k < V:
        keep = row_order(z)[:top_k]
    else:
        keep = np.arange(V)
    p = np.zeros(V)
    p[keep] = softmax(x[keep])
    if top_p < 1.0:
        order = keep[np.lexsort((keep, -p[keep]))]
        c = np.cumsum(p[order])
        n = int(np.searchsorted(c, top_p, side="left")) + 1
        n = max(1, min(n, len(order)))
        kept = order[:n]
        q = np.zeros(V)
        q[kept] = p[kept]
        p = q / q.sum()
    return p


def acceptance_probability(p: np.ndarray, q: np.ndarray) -> float:
    """Probability that d ~ q is accepted: sum_x q(x) min(1, p(x)/q(x)) = sum min(p, q)."""
    return float(np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum())


def inverse_cdf(weights: np.ndarray, u: float):
    """Smallest x with cumsum(w)[x] > u * sum(w); if rounding leaves none, the
    last x with w > 0.  Returns (x, margin): margin is the distance of u*sum(w)
    to the nearer of the two cumulative sums that bracket it."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    t = float(np.float64(u) * c[-1])
    x = int(np.searchsorted(c, t, side="right"))
    if x >= len(w):
        nz = np.nonzero(w > 0)[0]
        x = int(nz[-1]) if len(nz) else len(w) - 1
    lo = c[x - 1] if x > 0 else 0.0
    margin = min(abs(t - lo), abs(c[x] - t))
    return x, margin


def draw_weights(P_i: np.ndarray, Q_i=None) -> np.ndarray:
    """Weights of the replacement / extra draw at one position: max(0, P - Q)
    at a rejection (P itself if those all vanish), P alone when every draft
    was kept (Q_i is None)."""
    if Q_i is None:
        return np.asarray(P_i, dtype=np.float64)
    w = np.maximum(0.0, np.asarray(P_i, np.float64) - np.asarray(Q_i, np.float64))
    if w.sum() == 0.0:
        w = np.asarray(P_i, dtype=np.float64)
    return w


def cdf_distance(weights: np.ndarray, u: float, x: int) -> float:
    """Distance of u * sum(w) to token x's interval [cumsum(w)[x-1], cumsum(w)[x])
    of the inverse-CDF draw (0 when x is the token drawn; +inf for a token of
    zero weight, which the draw can never emit)."""
    w = np.asarray(weights, dtype=np.float64)
    if not (0 <= x < len(w)) or w[x] <= 0.0:
        return float("inf")
    c = np.cumsum(w)
    t = float(np.float64(u) * c[-1])
    lo = c[x - 1] if x > 0 else 0.0
    hi = c[x]
    if lo <= t < hi:
        return 0.0
    return float(min(abs(t - lo), abs(t - hi)))


def verify(z_target, z_draft, draft_tokens, uniforms, temperature: float,
           top_k: int = 0, top_p: float = 1.0, want_probs: bool = False):
    """Verify a batch of drafted blocks.

    z_target [B, G+1, V] fp32; z_draft [B, G, V] fp32 (unused when greedy);
    draft_tokens [B, G] int; uniforms [B, G+1, 2] fp32.
    Returns a dict with tau [B], out_tokens [B, G+1] (accepted drafts, then the
    replacement / extra token, then -1), accept_ratio [B, G] (fp32 ratio; greedy:
    1.0 on a match else 0.0), near_ties [B] (decisions taken within 1e-6),
    sample_margin [B], and with want_probs the probability rows.
    """
    z_target = np.asarray(z_target)
    B, G1, V = z_target.shape
    G = G1 - 1
    greedy = temperature == 0.0
    tau = np.zeros(B, dtype=np.int32)
    out = np.full((B, G + 1), -1, dtype=np.int32)
    ratio = np.zeros((B, G), dtype=np.float32)
    near = np.zeros(B, dtype=np.int32)
    margin = np.full(B, np.inf)
    probs_t = np.zeros((B, G + 1, V)) if want_probs else None
    probs_d = np.zeros((B, G, V)) if (want_probs and z_draft is not None) else None
    for b in range(B):
        d = np.asarray(draft_tokens[b], dtype=np.int64)
        if greedy:
            choice = [int(np.argmax(z_target[b, i])) for i in range(G + 1)]
            t = G
            for i in range(G):
                ratio[b, i] = 1.0 if d[i] == choice[i] else 0.0
            for i in range(G):
                if d[i] != choice[i]:
                    t = i
                    break
            tau[b] = t
            out[b, :t] = d[:t]
            out[b, t] = choice[t]
            margin[b] = np.inf
            if want_probs:
                for i in range(G + 1):
                    probs_t[b, i] = softmax(z_target[b, i])
                if probs_d is not None:
                    for i in range(G):
                        probs_d[b, i] = softmax(z_draft[b, i])
            continue
        P = [filtered_probs(z_target[b, i], temperature, top_k, top_p) for i in range(G + 1)]
        Q = [filtered_probs(z_draft[b, i], temperature, top_k, top_p) for i in range(G)]
        if want_probs:
            probs_t[b] = np.stack(P)
            if G:
                probs_d[b] = np.stack(Q)
        t = G
        with np.errstate(divide="ignore", invalid="ignore"):
            for i in range(G):
                p32 = np.float32(P[i][d[i]])
                q32 = np.float32(Q[i][d[i]])
                ratio[b, i] = np.float32(p32 / q32)
        for i in range(G):
            u = np.float32(uniforms[b, i, 0])
            r = ratio[b, i]
            if abs(float(u) - float(r)) < NEAR_TIE:
                near[b] += 1
            if not (u < r):
                t = i
                break
        tau[b] = t
        out[b, :t] = d[:t]
        w = draw_weights(P[t], Q[t] if t < G else None)
        x, mg = inverse_cdf(w, float(np.float32(uniforms[b, t, 1])))
        out[b, t] = x
        margin[b] = mg
        if mg < NEAR_TIE:
            near[b] += 1
    res = dict(tau=tau, out_tokens=out, accept_ratio=ratio, near_ties=near, sample_margin=margin)
    if want_probs:
        res["target_probs"] = probs_t
        res["draft_probs"] = probs_d
    return res


def confidence_label(p: np.ndarray, q: np.ndarray) -> float:
    """DSpark tutorial, confidence-scheduled verification: the label of a drafted
    position is one minus the total-variation distance of the draft and target
    distributions, which equals sum_x min(p, q) (the acceptance probability)."""
    return acceptance_probability(p, q)


def verify_ragged(z_target, z_draft, draft_tokens, uniforms, row_cu, temperature: float,
                  top_k: int = 0, top_p: float = 1.0, want_beta: bool = False):
    """Verify requests with their own drafted lengths (the per-request verify
    length the DSpark tutorial's prefix scheduler picks).

    Request b owns target rows row_cu[b] .. row_cu[b+1] - 1 (G_b + 1 of them)
    and draft rows row_cu[b] - b .. row_cu[b+1] - b - 2 (G_b).  z_target
    [N, V], z_draft [N - B, V], draft_tokens [N - B], uniforms [N, 2].
    Each request is verified exactly as verify() does for a batch of one.
    Returns tau [B], out_tokens [N], accept_ratio [N - B], sample_margin [B],
    near_ties [B] and, with want_beta, beta [N - B]: the confidence label of
    each drafted position under the verification distributions (greedy: the
    point masses at the two lowest-index maxima)."""
    row_cu = np.asarray(row_cu, dtype=np.int64)
    B = len(row_cu) - 1
    N = int(row_cu[-1])
    tau = np.zeros(B, dtype=np.int32)
    out = np.full(N, -1, dtype=np.int32)
    ratio = np.zeros(N - B, dtype=np.float32)
    margin = np.full(B, np.inf)
    near = np.zeros(B, dtype=np.int32)
    beta = np.zeros(N - B) if want_beta else None
    greedy = temperature == 0.0
    for b in range(B):
        t0, t1 = int(row_cu[b]), int(row_cu[b + 1])
        G = t1 - t0 - 1
        d0 = t0 - b
        zd = None if z_draft is None else np.asarray(z_draft[d0:d0 + G])[None]
        r = verify(np.asarray(z_target[t0:t1])[None], zd, np.asarray(draft_tokens[d0:d0 + G])[None],
                   None if uniforms is None else np.asarray(uniforms[t0:t1])[None], temperature, top_k, top_p)
        tau[b] = r["tau"][0]
        out[t0:t1] = r["out_tokens"][0]
        ratio[d0:d0 + G] = r["accept_ratio"][0]
        margin[b] = r["sample_margin"][0]
        near[b] = r["near_ties"][0]
        if want_beta:
            for i in range(G):
                if greedy:
                    beta[d0 + i] = float(np.argmax(z_target[t0 + i]) == np.argmax(z_draft[d0 + i]))
                else:
                    beta[d0 + i] = confidence_label(filtered_probs(z_target[t0 + i], temperature, top_k, top_p),
                                                    filtered_probs(z_draft[d0 + i], temperature, top_k, top_p))
    res = dict(tau=tau, out_tokens=out, accept_ratio=ratio, sample_margin=margin, near_ties=near)
    if want_beta:
        res["beta"] = beta
    return res
