"""SwiGLU expert FFN and the MoE layer output, float64.  (Oracle: test infrastructure only.)

An expert is three matrices, gate, up and down (explainer page, "The bus
problem": three projections of hidden x inter per expert; NVMe-streaming
page, "Workflow": a SwiGLU expert kernel), so FFN(x) = W_down (silu(W_gate x)
* (W_up x)) with silu(z) = z / (1 + e^-z).  The layer output is the sum over
the token's top-k picks of gate weight times the expert's FFN, plus, when the
model has one, the always-on shared expert with weight 1 (explainer page,
"The model that should not fit": 10 routed + 1 shared; 95 GiB page,
"Decode": shared experts stay resident).

The SGLang page ("Can paging change the model's outputs?") states that the
paged layer returns what the unpaged one does; the layer output is therefore
this plain definition, whatever cache state produced it.  A layer stack
chains layers through a residual, x_{l+1} = x_l + y_l (this project's
reading: a stack whose next-layer prefetch means something needs layer l+1's
input to depend on layer l).
"""
import numpy as np

from . import route as _route


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(x, w_gate, w_up, w_down):
    """x [..., H] -> [..., H]; weights float64 [I, H], [I, H], [H, I]."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ w_gate.T
    u = x @ w_up.T
    return (silu(g) * u) @ w_down.T


class ExpertSource:
    """Decoded experts, looked up by (layer, expert); decodes lazily and keeps a few."""

    def __init__(self, get_weights, keep=64):
        self.get = get_weights
        self.keep = keep
        self.memo = {}

    def __call__(self, layer, expert):
        key = (layer, int(expert))
        w = self.memo.get(key)
        if w is None:
            w = self.get(layer, int(expert))
            if len(self.memo) >= self.keep:
                self.memo.pop(next(iter(self.memo)))
            self.memo[key] = w
        return w


def moe_layer(x, w_r, top_k, experts, layer=0, shared=None):
    """Sparse MoE layer.

    x [b, H]; w_r [E, H]; experts(layer, e) -> (Wg, Wu, Wd) float64;
    shared: (Wg, Wu, Wd) or None.  Returns (y [b, H] float64, ids, gate).
    """
    x = np.asarray(x, dtype=np.float64)
    ids, gate, _z, _p = _route.route(x, w_r, top_k)
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(top_k):
            wg, wu, wd = experts(layer, ids[t, j])
            y[t] += gate[t, j] * expert_ffn(x[t], wg, wu, wd)
        if shared is not None:
            y[t] += expert_ffn(x[t], *shared)
    return y, ids, gate


def moe_layer_given_routing(x, ids, gate, experts, layer=0, shared=None):
    """Layer output for a routing that is checked separately: y[t] = sum over the picks j of
    token t, in rank order, of gate[t, j] * FFN_{ids[t, j]}(x[t]), plus FFN_shared(x[t]).

    x [b, H]; ids, gate [b, k]; experts(layer, e) -> (Wg, Wu, Wd) float64.  Each expert's
    FFN is evaluated once on the matrix of the token rows that picked it (the same values
    as one row at a time, a matrix product per expert instead of a vector product per
    pick, so that thousands of picks stay cheap); the weighted sum then runs per token over
    its picks in rank order.
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    gate = np.asarray(gate, dtype=np.float64)
    b, k = ids.shape
    f = np.zeros((b, k, x.shape[1]))               # FFN output of every pick
    for e in np.unique(ids):
        tt, jj = np.nonzero(ids == e)
        wg, wu, wd = experts(layer, int(e))
        f[tt, jj] = expert_ffn(x[tt], wg, wu, wd)
    y = np.zeros_like(x)
    for j in range(k):
        y += gate[:, j:j + 1] * f[:, j]
    if shared is not None:
        y += expert_ffn(x, *shared)
    return y


def moe_layer_dense(x, w_r, top_k, all_experts, shared=None):
    """Dense brute force: every expert's FFN, weighted by p if it is in the top-k else 0.

    all_experts: list of (Wg, Wu, Wd) for e = 0..E-1.
    """
    x = np.asarray(x, dtype=np.float64)
    z = _route.logits(x, w_r)
    p = _route.softmax(z)
    E = z.shape[1]
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        chosen = set(int(e) for e in _route.rank_order(z[t])[:top_k])
        for e in range(E):
            g = p[t, e] if e in chosen else 0.0
            y[t] += g * expert_ffn(x[t], *all_experts[e])
        if shared is not None:
            y[t] += expert_ffn(x[t], *shared)
    return y
