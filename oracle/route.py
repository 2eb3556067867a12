"""Router of the MoE layer, float64.  (Oracle: test infrastructure only.)

Explainer page, "The model that should not fit": a small router reads each
token and picks a few experts; the SGLang page, "What does Paged Experts
actually do?": each token goes to top_k of E experts.  Readings fixed here
(the pages leave them open):

* logits z = W_r x, softmax p = exp(z - max z) / sum exp(z - max z);
* the top-k is taken on z (softmax is monotone), in rank order: descending z,
  equal z broken by the lower expert index;
* the gate weight of a pick is p of that expert, NOT renormalised over the
  k picks (no page mentions renormalisation);
* near ties: two ranks inside the top k+1 whose logits differ by at most
  tau = 1e-10 * (1 + sum_i |W_r[e, i] x_i|) (larger of the two experts) may
  come out in either order from two correct float64 evaluations with
  different summation orders; ``near_ties`` lists them.
"""
import numpy as np


def logits(x, w_r):
    """x [b, H], w_r [E, H] -> z [b, E] float64 (plain float64 matrix product)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_r, dtype=np.float64).T


def softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def rank_order(z_row):
    """Expert indices of one token sorted by descending logit, ties by ascending index."""
    idx = np.arange(z_row.shape[0])
    return np.lexsort((idx, -z_row))


def route(x, w_r, top_k):
    """Returns (ids [b, k] int64 in rank order, gate [b, k] float64, z [b, E], p [b, E])."""
    z = logits(x, w_r)
    p = softmax(z)
    b = z.shape[0]
    ids = np.empty((b, top_k), dtype=np.int64)
    for t in range(b):
        ids[t] = rank_order(z[t])[:top_k]
    gate = np.take_along_axis(p, ids, axis=1)
    return ids, gate, z, p


def abs_mass(x, w_r):
    """A[t, e] = sum_i |W_r[e, i] x_i|, the scale of the float64 summation error of z[t, e]."""
    return np.abs(np.asarray(x, dtype=np.float64)) @ np.abs(np.asarray(w_r, dtype=np.float64)).T


def near_ties(z, amass, top_k, rel=1e-10):
    """[(t, r)] where ranks r and r+1 (r < top_k) of token t are within tau of each other."""
    out = []
    for t in range(z.shape[0]):
        order = rank_order(z[t])
        for r in range(min(top_k, z.shape[1] - 1)):
            a, b = order[r], order[r + 1]
            tau = rel * (1.0 + max(amass[t, a], amass[t, b]))
            if z[t, a] - z[t, b] <= tau:
                out.append((t, r))
    return out


def ids_match_with_ties(ids_ref, ids_other, z, amass, rel=1e-10):
    """True if ids_other equals ids_ref up to swaps of near-tied adjacent picks.

    Both must hold the same top-k set apart from a near-tie at the k-th
    boundary; every position where they differ must be explained by a
    near tie (logit gap <= tau) between the two experts involved.
    """
    ids_ref = np.asarray(ids_ref)
    ids_other = np.asarray(ids_other)
    for t in range(ids_ref.shape[0]):
        if np.array_equal(ids_ref[t], ids_other[t]):
            continue
        for a, b in zip(ids_ref[t], ids_other[t]):
            if a == b:
                continue
            tau = rel * (1.0 + max(amass[t, a], amass[t, b]))
            if abs(z[t, a] - z[t, b]) > tau:
                return False
    return True
