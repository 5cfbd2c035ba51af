"""Sampling controls: logit bias, repetition / presence / frequency penalties,
temperature, top-k, top-p, min-p, and the draw -- oracle, test
infrastructure.

"MoE-Xtend" README, SAMPLING CONTROLS: p = softmax(z / T); top-k keeps the k
most probable tokens; top-p keeps the smallest set whose cumulative
probability reaches p; min-p drops the tokens whose probability is below a
fraction of the most probable token's; logit bias comes first, then the
repetition, presence and frequency penalties, then the truncations (top-k,
top-p, min-p), then the draw; temperature 0 decodes greedily.  The project
summary page: sampling is deterministic.  GPT-OSS-Lite README, model
diagram: a vocabulary of 128,000 tokens.

Readings (the pages name the controls, not their formulas):
  * the logits are fp32 (an fp32 model head's output); bias, then the
    penalties are elementwise fp32 operations in the order named:
      z <- z + bias;
      repetition r (1 = off), for a token seen c_v > 0 times:
        z <- z / r if z > 0, else z * r;
      presence a (0 = off):  z <- z - a [c_v > 0];
      frequency f (0 = off): z <- z - f c_v   (the product rounded, then
                                              the difference);
    c_v counts the token's occurrences in the sequence so far;
  * greedy (T = 0): the largest processed logit, ties to the lower id;
  * a truncation never splits a group of equally probable tokens: top-k
    keeps every token at least as probable as the k-th most probable one
    (k = 0 or k >= V: off); top-p, taken on the top-k set renormalised,
    keeps every token at least as probable as the one at which the
    cumulative share, summed in decreasing probability, first reaches p
    (p = 1: off); min-p keeps the tokens with p >= min_p * max p (0: off);
    the kept set is the intersection of the three (each is a probability
    threshold, so the tightest one decides);
  * the draw takes one uniform u in [0, 1) per row as input (the only
    random number) and inverts the kept distribution in increasing token
    id: the first kept token whose cumulative share of the kept mass
    exceeds u;
  * a row whose processed logits are all -inf has no token: -1.
"""
import numpy as np


def processed_logits(z, bias, counts, rep, presence, frequency):
    """z [V] fp32 logits, bias [V] or None, counts [V] int -> fp32 [V]."""
    z = np.asarray(z, np.float32).copy()
    if bias is not None:
        z = z + np.asarray(bias, np.float32)
    c = np.asarray(counts, np.int64)
    seen = c > 0
    r = np.float32(rep)
    z = np.where(seen, np.where(z > 0, z / r, z * r), z).astype(np.float32)
    z = np.where(seen, z - np.float32(presence), z).astype(np.float32)
    fc = (np.float32(frequency) * c.astype(np.float32)).astype(np.float32)
    return (z - fc).astype(np.float32)


def token_counts(history, V):
    """history: token ids, entries outside [0, V) ignored -> counts [V]."""
    h = np.asarray(history, np.int64).ravel()
    h = h[(h >= 0) & (h < V)]
    return np.bincount(h, minlength=V)


def probabilities(zp, temperature):
    """softmax(zp / T) in fp64 (T > 0)."""
    s = np.asarray(zp, np.float64) / float(temperature)
    e = np.exp(s - s.max())
    return e / e.sum()


def kept_mask(zp, temperature, top_k, top_p, min_p):
    """Boolean mask of the tokens the three truncations keep."""
    zp = np.asarray(zp, np.float32)
    V = zp.size
    p = probabilities(zp, temperature)
    keep = np.ones(V, bool)
    if 0 < top_k < V:
        vk = np.sort(zp)[::-1][top_k - 1]          # the k-th largest, with multiplicity
        keep &= zp >= vk
    if top_p < 1.0:
        order = np.argsort(-zp[keep], kind="stable")
        ids = np.flatnonzero(keep)[order]
        share = np.cumsum(p[ids]) / p[ids].sum()
        j = int(np.argmax(share >= top_p)) if np.any(share >= top_p) else len(ids) - 1
        keep &= zp >= zp[ids[j]]
    if min_p > 0.0:
        keep &= p >= min_p * p.max()
    return keep


def sample(z, bias, counts, rep, presence, frequency, temperature, top_k, top_p, min_p, u):
    """One row: (token id, processed logits, kept mask or None)."""
    zp = processed_logits(z, bias, counts, rep, presence, frequency)
    if not np.any(zp > -np.inf):
        return -1, zp, None
    if temperature == 0.0:
        return int(np.argmax(zp)), zp, None          # np.argmax takes the first of equals
    keep = kept_mask(zp, temperature, top_k, top_p, min_p)
    p = probabilities(zp, temperature)
    ids = np.flatnonzero(keep)
    cum = np.cumsum(p[ids]) / p[ids].sum()
    i = min(int(np.searchsorted(cum, u, side="right")), len(ids) - 1)
    return int(ids[i]), zp, keep
