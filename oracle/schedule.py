"""Oracle of the hardware-aware prefix scheduler (test infrastructure only).

DSpark tutorial, confidence-scheduled verification, "hardware-aware prefix
scheduler": given a pool of requests, each drafted position carrying a
conditional survival probability c_k (the chance it passes verification
when everything before it passed), choose each request's verify length
ell_r to maximise the throughput Theta = tau * SPS(B), where B is the total
number of verified tokens and SPS(B) a measured batch -> steps-per-second
curve.  The greedy: sort every request's candidate tokens by cumulative
survival prod_{i <= k} c_i, descending; extend verify lengths one token at a
time in that order, recomputing Theta; stop at the first token that does not
raise it.

Readings taken where the page leaves a step open:
  * a request verifying ell_r drafted tokens puts ell_r + 1 tokens into the
    verify batch (its last accepted token plus the drafts), so
    B = sum_r (ell_r + 1);
  * tau is the expected number of tokens the step emits: each request emits
    its correction / extra token plus the expected accepted prefix,
    tau = sum_r (1 + sum_{k <= ell_r} prod_{i <= k} c_{r,i});
  * SPS(B) is the piecewise-linear interpolation of the table (B_j, s_j)
    (sorted by B), clamped to the end values outside it;
  * ties in cumulative survival go to the lower request index, then the
    lower position, so every request's lengths grow as prefixes;
  * "does not raise" means Theta' <= Theta (strict improvement to go on).
"""
import numpy as np


def sps_interp(B: float, table_b, table_v) -> float:
    """Steps per second at verify batch B from the measured table."""
    tb = np.asarray(table_b, dtype=np.float64)
    tv = np.asarray(table_v, dtype=np.float64)
    return float(np.interp(float(B), tb, tv))


def prefix_schedule(survival, table_b, table_v):
    """survival: list over requests of arrays of conditional survival
    probabilities c_{r,1..L_r}.  Returns (ell [R] int, theta float)."""
    R = len(survival)
    cum = [np.cumprod(np.asarray(c, dtype=np.float64)) for c in survival]
    cands = [(-float(cum[r][k]), r, k + 1) for r in range(R) for k in range(len(cum[r]))]
    cands.sort()
    ell = np.zeros(R, dtype=np.int64)
    B = R
    tau = float(R)
    theta = tau * sps_interp(B, table_b, table_v)
    for neg_s, r, k in cands:
        if k != ell[r] + 1:
            continue
        tau2 = tau + (-neg_s)
        th2 = tau2 * sps_interp(B + 1, table_b, table_v)
        if not th2 > theta:
            break
        ell[r] = k
        B += 1
        tau = tau2
        theta = th2
    return ell, theta
