"""The two-level oracle evaluated on sampled elements of a long buffer.

A ring level starts element i's chunk at member (i // L) mod m, with L the
level's chunk length and m its member count, and then runs through the
members in order.  Rotating every node's peers by the local start and the
nodes by the global start, and running the oracle on that one-element
column (whose chunks all start at member 0), therefore gives element i the
association the whole-buffer oracle would give it.  Tree and centralized
levels have a fixed order and are not rotated.  The CPU tests check this
against the whole-buffer oracle on short buffers."""

import numpy as np

import oracle


def _starts(idx, n, members, strategy):
    name, param = strategy
    if name != "ring":
        return np.zeros(len(idx), dtype=np.int64)
    chunks = param if param else members
    L = -(-n // chunks)
    return (np.asarray(idx, dtype=np.int64) // L) % members


def hierarchical_sampled(V, idx, n, op, nodes, local, global_, in_dtype="f32", out_dtype=None):
    """V: (P, len(idx)) values of the sampled elements of an n-element
    buffer (bf16 as bit patterns); returns (P, len(idx)) results."""
    P = V.shape[0]
    G = int(nodes)
    Lr = P // G
    s_l = _starts(idx, n, Lr, local)
    s_g = _starts(idx, n, G, global_)
    out = None
    for c in range(V.shape[1]):
        col = np.empty((P, 1), dtype=V.dtype)
        for g in range(G):
            for l in range(Lr):
                col[g * Lr + l, 0] = V[((g + s_g[c]) % G) * Lr + (l + s_l[c]) % Lr, c]
        y = oracle.hierarchical_allreduce(col, op, nodes=G, local=local, global_=global_,
                                          in_dtype=in_dtype, out_dtype=out_dtype)
        if out is None:
            out = np.empty((P, V.shape[1]), dtype=y.dtype)
        out[:, c] = y[:, 0]
    return out
