"""Sink-augmented grouped-query attention in fp64 -- oracle, test infrastructure.

Definition (plain form, no online softmax, no blocking):

  * GQA ("GQA Attention" study note, "How it works"): q_mult = n_q / n_kv;
    query head h = g*q_mult + m belongs to KV head g = h // q_mult; keys and
    values are shared inside a group, sinks and queries are not.
  * score ("MoE-Xtend" README, ATTENTION STACK; study note, "How it works"):
    l_j = sm_scale * <q, k_j> + M_j, M_j in {0, -inf}.
  * masks ("MoE-Xtend" README, ATTENTION STACK, mask engineering), for a query
    at global position p = offset + t and key row j of the cache:
        causal: allowed iff j <= p
        band of width W: the README writes j >= p - W (W+1 keys) while the
        study note writes p - W < j <= p (W keys).  This oracle takes the
        study note's reading, W keys including the diagonal, which matches
        the "128-token window" both pages name.  W <= 0 means no band.
  * sink ("MoE-Xtend" README, ATTENTION STACK, sink bias; study note): one
    learned logit sigma_h per query head is appended as an extra softmax
    column and dropped after normalisation:
        out = sum_j exp(l_j - M) v_j / (exp(sigma_h - M) + sum_j exp(l_j - M)),
        M = max(sigma_h, max_j l_j).
    sigma is in scaled-logit units (not multiplied by sm_scale), carries no
    RoPE, and sigma = -inf gives a plain causal / band softmax.

Two forms are given: ``attend_query`` / ``sink_attention`` walk query by
query over the allowed key range; ``sink_attention_dense`` writes the
definition out with a dense [T, n_ctx] additive mask matrix built against the
cache width, expanded K/V, a concatenated sink column, a full softmax and the
column dropped.  The tests hold the two against each other.
"""
import numpy as np


def allowed_range(p: int, window: int):
    """Half-open key range [lo, hi) allowed for a query at position p."""
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, p + 1


def attend_query(q_heads: np.ndarray, Kc: np.ndarray, Vc: np.ndarray,
                 sinks: np.ndarray, p: int, window: int,
                 sm_scale: float) -> np.ndarray:
    """All n_q heads of one query token at global position p.

    q_heads [n_q, d] (already rotated); Kc, Vc [rows, n_kv, d] one sequence's
    cache; sinks [n_q].  Returns fp64 [n_q, d]."""
    n_q, d = q_heads.shape
    n_kv = Kc.shape[1]
    q_mult = n_q // n_kv
    lo, hi = allowed_range(p, window)
    out = np.empty((n_q, d), dtype=np.float64)
    for g in range(n_kv):
        hs = slice(g * q_mult, (g + 1) * q_mult)
        Q = np.asarray(q_heads[hs], dtype=np.float64)          # [q_mult, d]
        K = np.asarray(Kc[lo:hi, g], dtype=np.float64)         # [n, d]
        V = np.asarray(Vc[lo:hi, g], dtype=np.float64)
        sig = np.asarray(sinks[hs], dtype=np.float64)          # [q_mult]
        logits = sm_scale * (Q @ K.T)                          # [q_mult, n]
        M = np.maximum(sig, logits.max(axis=1))
        e = np.exp(logits - M[:, None])
        Z = np.exp(sig - M) + e.sum(axis=1)
        out[hs] = (e @ V) / Z[:, None]
    return out


def sink_attention(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray,
                   sinks: np.ndarray, q_offset: int, window: int,
                   sm_scale: float) -> np.ndarray:
    """q [B, T, n_q, d] at positions q_offset + t; Kc, Vc [B, rows, n_kv, d].

    Rows past the last query position are never read (causal mask)."""
    B, T, n_q, d = q.shape
    if n_q % Kc.shape[2]:
        raise ValueError("n_q must be a multiple of n_kv")
    out = np.empty((B, T, n_q, d), dtype=np.float64)
    for b in range(B):
        for t in range(T):
            out[b, t] = attend_query(q[b, t], Kc[b], Vc[b], sinks,
                                     q_offset + t, window, sm_scale)
    return out


def mask_matrix(T: int, n_ctx: int, offset: int, window: int) -> np.ndarray:
    """Additive mask [T, n_ctx]: causal plus (for window > 0) the band."""
    qi = np.arange(T)[:, None]
    kj = np.arange(n_ctx)[None, :]
    causal = np.where(kj <= offset + qi, 0.0, -np.inf)
    if window > 0:
        band = np.where(kj > offset + qi - window, 0.0, -np.inf)
    else:
        band = np.zeros((T, n_ctx))
    return causal + band


def sink_attention_dense(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray,
                         sinks: np.ndarray, q_offset: int, window: int,
                         sm_scale: float) -> np.ndarray:
    """The definition written out with a dense mask matrix (tiny shapes).

    The mask is built against the full cache width n_ctx = Kc.shape[1]; cache
    rows must be finite (masked rows get weight exactly 0)."""
    B, T, n_q, d = q.shape
    n_ctx, n_kv = Kc.shape[1], Kc.shape[2]
    q_mult = n_q // n_kv
    K = np.repeat(np.asarray(Kc, dtype=np.float64), q_mult, axis=2)  # [B, n_ctx, n_q, d]
    V = np.repeat(np.asarray(Vc, dtype=np.float64), q_mult, axis=2)
    Q = np.asarray(q, dtype=np.float64)
    S = np.einsum("bthd,bjhd->bhtj", Q, K) * sm_scale
    S = S + mask_matrix(T, n_ctx, q_offset, window)[None, None]
    sink_col = np.broadcast_to(np.asarray(sinks, np.float64)[None, :, None, None],
                               (B, n_q, T, 1))
    S_aug = np.concatenate([S, sink_col], axis=-1)
    S_aug = S_aug - S_aug.max(axis=-1, keepdims=True)
    W = np.exp(S_aug)
    W = W / W.sum(axis=-1, keepdims=True)
    W = W[..., :-1]                                  # drop the sink column
    return np.einsum("bhtj,bjhd->bthd", W, V)
