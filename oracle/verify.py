"""Full-vocabulary verification and the DLoop gate -- oracle.

Test infrastructure: see the package header for who may import this.

Greedy acceptance follows [SGLang DFlash, section 3, the function that computes
the correct drafts and the bonus]: draft token i+1 of the candidates (i.e.
draft i here) is compared with the target's prediction at row i; the accepted
length is the number of leading matches (cumulative product of the matches,
summed); the bonus token is the target prediction at row accept_len; the
committed length is accept_len + 1.  The target prediction of a row is its
argmax over the vocabulary.

Sampled acceptance follows [Spec-decoding tutorial, section 3]: draft token x
at row i is kept with probability min(1, p_i(x)/q_i(x)); at the first
rejection the replacement is drawn from the residual max(0, p - q)
normalised by 1 - beta with beta = sum_y min(p(y), q(y)); [section 4]: later
drafts are discarded; and [DFlash overview, "关键伪代码"]: when every draft is
accepted the bonus is drawn from the target distribution of the last row.
[DLoop, "验证与无损性"]: several drafted stages are verified as one chain with
the ordinary per-position rule (one chain, one bonus).

The gate follows [DLoop, "机制一：置信度门控", the equations for c_s and
f_gate]: c_s is the sum over the stage's drafted tokens of the drafter's log
probability of each token, and drafting continues iff c_s >= g.

Readings where the pages leave a step open (also in the design doc):
* argmax ties go to the lowest token id; an all -inf row has argmax 0;
* randomness enters only through caller-supplied uniforms: u[b, i] decides
  row i (accept iff u < p/q, strict; q(x) = 0 accepts), u'[b] draws the bonus
  by inverse CDF in ascending token order: the smallest x whose cumulative
  weight exceeds u' * (total weight), strictly; if rounding leaves no such x,
  the last x with positive weight;
* the residual is normalised by its own computed sum R (equal to 1 - beta in
  exact arithmetic); if R == 0 the bonus is drawn from p of that row;
* p and q are softmax(logits / T) with the same temperature T > 0;
* a request's chain length n_b <= L limits the rows used: target rows
  0..n_b, draft rows 0..n_b-1;
* a draft token outside [0, V) among the first n_b makes the request an
  in-band error: accept_len = bonus = -1, commit = 0, new_seq_len = prefix;
* the gate sums only drafted tokens (the anchor is not drafted) and uses the
  sampling temperature; a tie c == g continues.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .numerics import widen


def _first_argmax(row):
    """Lowest index attaining the maximum."""
    best = row.max()
    return int(np.flatnonzero(row == best)[0])


def _softmax(x):
    m = x.max()
    e = np.exp(x - m)
    return e / e.sum()


def _logsumexp(x):
    m = x.max()
    return m + np.log(np.exp(x - m).sum())


def row_log_softmax(x):
    return x - _logsumexp(x)


def _lens(chain_lens, B, L):
    return np.full(B, L, dtype=np.int64) if chain_lens is None else np.asarray(chain_lens)


@dataclass
class GreedyResult:
    accept_len: np.ndarray      # [B] int
    bonus: np.ndarray           # [B] int
    commit_lens: np.ndarray     # [B] int
    new_seq_lens: Optional[np.ndarray]
    target_predict: np.ndarray  # [B, L+1], -1 where the row is past the chain
    draft_tokens: np.ndarray    # [B, L], -1 where past the chain


def verify_greedy(target_logits, dtype, draft_tokens=None, draft_logits=None,
                  chain_lens=None, prefix_lens=None) -> GreedyResult:
    t = widen(target_logits, dtype)
    B, Lp1, V = t.shape
    L = Lp1 - 1
    n = _lens(chain_lens, B, L)
    tp = np.full((B, L + 1), -1, dtype=np.int64)
    dt = np.full((B, L), -1, dtype=np.int64)
    d = None if draft_logits is None else widen(draft_logits, dtype)
    acc = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    for b in range(B):
        nb = int(n[b])
        for i in range(nb + 1):
            tp[b, i] = _first_argmax(t[b, i])
        for i in range(nb):
            dt[b, i] = _first_argmax(d[b, i]) if d is not None else int(draft_tokens[b, i])
        if np.any((dt[b, :nb] < 0) | (dt[b, :nb] >= V)):
            acc[b] = bonus[b] = -1
            continue
        a = 0
        while a < nb and dt[b, a] == tp[b, a]:
            a += 1
        acc[b] = a
        bonus[b] = tp[b, a]
    commit = np.where(acc >= 0, acc + 1, 0)
    new = None if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64) + commit
    return GreedyResult(acc, bonus, commit, new, tp, dt)


@dataclass
class SampleResult:
    accept_len: np.ndarray
    bonus: np.ndarray
    commit_lens: np.ndarray
    new_seq_lens: Optional[np.ndarray]
    ratio: np.ndarray         # [B, L] p/q at the rows tested, NaN elsewhere
    beta: np.ndarray          # [B] sum min(p, q) of the rejected row, NaN if none
    cdf_gap: np.ndarray       # [B] distance of u'*Z to the nearest CDF boundary / Z
    ratio_gap: np.ndarray     # [B] min |u - ratio| over the rows tested
    bonus_row: np.ndarray     # [B] row the bonus came from
    rejected: np.ndarray      # [B] bool


def _inverse_cdf(w, u):
    """Smallest x with cumsum(w)[x] > u * sum(w); fallback: last x with w > 0.
    Also returns the gap of u*Z to the nearer bracketing boundary, over Z."""
    c = np.cumsum(w)
    Z = c[-1]
    thr = u * Z
    hit = np.flatnonzero(c > thr)
    if hit.size:
        x = int(hit[0])
    else:
        x = int(np.flatnonzero(w > 0)[-1])
    lo = c[x - 1] if x > 0 else 0.0
    gap = min(abs(thr - lo), abs(c[x] - thr)) / Z if Z > 0 else 0.0
    return x, gap


def residual(target_row, draft_row):
    """One row pair's acceptance quantities ([Spec-decoding tutorial], section 3):
    p = softmax(target_row), q = softmax(draft_row) (both already divided by the
    temperature), the overlap min(p, q) whose sum is beta, and the residual
    max(0, p - q) whose sum R equals 1 - beta in exact arithmetic."""
    p, q = _softmax(target_row), _softmax(draft_row)
    return p, q, np.minimum(p, q), np.maximum(0.0, p - q)


def verify_sample(target_logits, draft_logits, draft_tokens, u_accept, u_bonus, dtype,
                  temperature=1.0, chain_lens=None, prefix_lens=None) -> SampleResult:
    t = widen(target_logits, dtype) / temperature
    d = widen(draft_logits, dtype) / temperature
    B, Lp1, V = t.shape
    L = Lp1 - 1
    n = _lens(chain_lens, B, L)
    acc = np.zeros(B, dtype=np.int64)
    bonus = np.zeros(B, dtype=np.int64)
    ratio = np.full((B, L), np.nan)
    beta = np.full(B, np.nan)
    cgap = np.full(B, np.nan)
    rgap = np.full(B, np.inf)
    brow = np.zeros(B, dtype=np.int64)
    rej = np.zeros(B, dtype=bool)
    for b in range(B):
        nb = int(n[b])
        toks = np.asarray(draft_tokens[b, :nb], dtype=np.int64)
        if np.any((toks < 0) | (toks >= V)):
            acc[b] = bonus[b] = -1
            continue
        a = nb
        for i in range(nb):
            x = toks[i]
            p, q = _softmax(t[b, i]), _softmax(d[b, i])
            r = p[x] / q[x] if q[x] > 0 else np.inf
            ratio[b, i] = r
            rgap[b] = min(rgap[b], abs(float(u_accept[b, i]) - r))
            if not (u_accept[b, i] < r):
                a = i
                rej[b] = True
                break
        acc[b] = a
        brow[b] = a
        if rej[b]:
            p, _, overlap, res = residual(t[b, a], d[b, a])
            beta[b] = overlap.sum()
            w = res if res.sum() > 0 else p
        else:
            w = _softmax(t[b, nb])
        bonus[b], cgap[b] = _inverse_cdf(w, float(u_bonus[b]))
    commit = np.where(acc >= 0, acc + 1, 0)
    new = None if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64) + commit
    return SampleResult(acc, bonus, commit, new, ratio, beta, cgap, rgap, brow, rej)


@dataclass
class GateResult:
    c: np.ndarray         # [B]
    go: np.ndarray        # [B] bool
    row_max: np.ndarray   # [B, n] max of logits / T
    row_lse: np.ndarray   # [B, n] logsumexp of logits / T


def gate(draft_logits, draft_tokens, dtype, temperature=1.0, g=-0.5,
         valid_lens=None) -> GateResult:
    d = widen(draft_logits, dtype) / temperature
    B, n, V = d.shape
    vl = _lens(valid_lens, B, n)
    c = np.zeros(B)
    rmax = np.zeros((B, n))
    rlse = np.zeros((B, n))
    for b in range(B):
        for i in range(n):
            rmax[b, i] = d[b, i].max()
            rlse[b, i] = _logsumexp(d[b, i])
        for i in range(int(vl[b])):
            c[b] += d[b, i, int(draft_tokens[b, i])] - rlse[b, i]
    return GateResult(c, c >= g, rmax, rlse)
