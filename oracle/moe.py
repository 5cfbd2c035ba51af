"""MoE layer: top-k router, dispatch by expert, the selected SwiGLU experts and
the weighted combine -- oracle, test infrastructure.

"MoE-Xtend" README, MOE ROUTING (canonical equations, batched view,
pseudocode, implementation notes): router logits S = X W_r^T [N, E]; the
top-k expert ids I per token; weights w = softmax over the k selected logits
only; y = sum over i in I of w_i E_i(x); the batched form groups token rows
by expert id and evaluates only the selected experts; floating-point ties in
top-k must be broken consistently or outputs become unstable.
"GPT-OSS-Lite" visual guide, Architecture Specifications: 8 routed experts,
2 active per token, 1 shared expert, SwiGLU experts with ffn_dim 1536,
d_model 768; the README's layer diagram: residual -> RMSNorm -> MoE (top-2
of 8) -> residual; its file list names a fused W1/W3 + SiLU dispatch.

Readings (the pages give the equations, not the precisions or the expert's
exact form):
  * the router is a bf16 linear layer without bias (the equation has none):
    logits = x W_r^T rounded once to bf16, and top-k runs on those bf16
    values, so ties are real; a tie goes to the lower expert index (the
    consistent tie-break the notes ask for);
  * the k selected logits are normalised by a softmax (fp64 here);
  * an expert is SwiGLU: E(x) = W2 (silu(W1 x) * (W3 x)), silu(a) = a / (1 +
    e^-a), each linear a bf16 layer without bias (rounded once), the gated
    product rounded to bf16 as it feeds the last bf16 linear;
  * the shared expert is one more SwiGLU expert applied to every token with
    weight 1;
  * y = sum_i w_i E_i(x) (+ shared) summed exactly and rounded once to bf16;
  * dispatch lists the (token, slot) pairs of each expert in token order.
"""
import numpy as np

from .rounding import round_to


def router_logits(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    """x [N, d_model], Wr [E, d_model] -> bf16 logits [N, E] (as float64)."""
    return round_to(np.asarray(x, np.float64) @ np.asarray(Wr, np.float64).T, "bf16")


def topk_stable(S: np.ndarray, k: int) -> np.ndarray:
    """[N, E] -> [N, k] expert ids, largest logit first, equal logits in
    increasing expert index."""
    N, E = S.shape
    idx = np.empty((N, k), dtype=np.int64)
    for t in range(N):
        order = sorted(range(E), key=lambda e: (-S[t, e], e))
        idx[t] = order[:k]
    return idx


def softmax_selected(S: np.ndarray, I: np.ndarray) -> np.ndarray:
    """Softmax over the k selected logits of each token -> [N, k] fp64."""
    sel = np.take_along_axis(np.asarray(S, np.float64), I, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def dispatch(I: np.ndarray, E: int):
    """Group the (token, slot) pairs by expert: returns (tokens, slots,
    start) with start [E+1] the first row of each expert; inside an expert
    the rows follow token order."""
    N, k = I.shape
    tokens, slots, start = [], [], [0]
    for e in range(E):
        for t in range(N):
            for s in range(k):
                if I[t, s] == e:
                    tokens.append(t)
                    slots.append(s)
        start.append(len(tokens))
    return np.array(tokens, np.int64), np.array(slots, np.int64), np.array(start, np.int64)


def silu(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, np.float64)
    return a / (1.0 + np.exp(-a))


def swiglu_expert(x: np.ndarray, W1: np.ndarray, W3: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """x [n, d_model], W1 and W3 [ffn, d_model], W2 [d_model, ffn] -> bf16
    output [n, d_model] (as float64), every bf16 linear rounded once."""
    x = np.asarray(x, np.float64)
    a = round_to(x @ np.asarray(W1, np.float64).T, "bf16")
    b = round_to(x @ np.asarray(W3, np.float64).T, "bf16")
    h = round_to(silu(a) * b, "bf16")
    return round_to(h @ np.asarray(W2, np.float64).T, "bf16")


def moe_layer(x, Wr, W1, W3, W2, k, shared=None, I=None):
    """x [N, d_model]; Wr [E, d_model]; W1, W3 [E, ffn, d_model]; W2 [E,
    d_model, ffn]; shared = (W1s, W3s, W2s) or None.  I: routing to use
    instead of the router's own (to evaluate the rest of the layer on a
    given routing).  Returns (y bf16 [N, d_model], S, I, w)."""
    S = router_logits(x, Wr)
    if I is None:
        I = topk_stable(S, k)
    w = softmax_selected(S, I)
    E = Wr.shape[0]
    tokens, slots, start = dispatch(I, E)
    acc = np.zeros((x.shape[0], x.shape[1]), np.float64)
    for e in range(E):
        rows = slice(start[e], start[e + 1])
        if start[e + 1] == start[e]:
            continue
        t, s = tokens[rows], slots[rows]
        out = swiglu_expert(x[t], W1[e], W3[e], W2[e])
        acc[t] += w[t, s][:, None] * out
    if shared is not None:
        acc += swiglu_expert(x, *shared)
    return round_to(acc, "bf16"), S, I, w
