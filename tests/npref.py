"""Second formulations used to pin the oracle (tests only).

These are written independently of ``oracle/moe_oracle.c``: NumPy float64 with
BLAS matrix products (a different summation order), bit-level roundings, full
sorts instead of arg-max passes, and an evaluation over the (token, expert) pairs
ordered by expert with a scatter-add back to the tokens instead of per-token
evaluation. They agree with the oracle to rounding order, not bit for bit.
"""
import numpy as np
import scipy.special


def widen(a, dt):
    """bf16 bits (uint16) or float32 -> float64."""
    if dt == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16_bits(x):
    """float64 -> bf16 value (as float64), round to nearest even, by integer ops on the
    float64 bit pattern: keep sign, exponent and 7 fraction bits (valid for normal bf16)."""
    x = np.asarray(x, np.float64)
    b = x.view(np.uint64).copy()
    low = np.uint64(45)  # 52 - 7 fraction bits dropped
    keep_lsb = (b >> low) & np.uint64(1)
    b = b + (np.uint64((1 << 44) - 1) + keep_lsb)
    b = b & ~np.uint64((1 << 45) - 1)
    return b.view(np.float64)


def round_f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def topk_by_sort(v, K):
    """Top-K of each row by a full stable sort on (-v, index); ids ascending."""
    n, E = v.shape
    out = np.empty((n, K), np.int64)
    for t in range(n):
        order = np.lexsort((np.arange(E), -v[t]))
        out[t] = np.sort(order[:K])
    return out


def swiglu_ffn(x, w1, w3, w2, hround):
    """x [n,d] float64; w1,w3 [I,d]; w2 [d,I] -> y [n,d]; H rounded by `hround`."""
    a = x @ w1.T
    g = x @ w3.T
    h = hround(a * sigmoid(a) * g)
    return h @ w2.T


def dense_layer(u, e, b, routed, shared, K, hround, score="sigmoid"):
    """All-experts dense evaluation: every routed expert on every token, with a gate
    matrix that is zero outside each token's top-K. Inputs are float64.
    score "sigmoid": top-K of sigmoid(z) + b, gates sigmoid(z) normalised; "softmax": top-K
    of z, gates scipy's softmax of the selected logits."""
    z = u @ e.T
    G = np.zeros_like(z)
    if score == "softmax":
        sel = topk_by_sort(z, K)
        for t in range(u.shape[0]):
            G[t, sel[t]] = scipy.special.softmax(z[t, sel[t]])
    else:
        s = sigmoid(z)
        sel = topk_by_sort(s + b[None, :], K)
        for t in range(u.shape[0]):
            G[t, sel[t]] = s[t, sel[t]]
            G[t] /= G[t, sel[t]].sum()
    out = u.copy()
    for (w1, w3, w2) in shared:
        out = out + swiglu_ffn(u, w1, w3, w2, hround)
    for i in range(e.shape[0]):
        out = out + G[:, i:i + 1] * swiglu_ffn(u, *routed[i], hround)
    return out, sel, G


def pair_scatter_layer(u, sel, gates, routed, shared, hround):
    """h'_t of the method's equation built from the (token, expert, gate) pairs: the T*K
    pairs are ordered by expert with a stable argsort, each expert's run of pairs is
    evaluated as one batch of FFN rows, and every row is scattered into its token's
    output with its gate (np.add.at adds the rows of one token in pair order). The shared
    experts and the residual complete the sum."""
    n, K = sel.shape
    tok = np.repeat(np.arange(n), K)
    ex = np.asarray(sel).reshape(-1)
    g = np.asarray(gates, np.float64).reshape(-1)
    order = np.argsort(ex, kind="stable")
    ex_sorted = ex[order]
    starts = np.flatnonzero(np.r_[True, ex_sorted[1:] != ex_sorted[:-1]])
    ends = np.r_[starts[1:], ex_sorted.size]
    rows = np.empty((ex.size, u.shape[1]))
    for a, z in zip(starts, ends):
        p = order[a:z]
        rows[p] = swiglu_ffn(u[tok[p]], *routed[int(ex_sorted[a])], hround)
    routed_out = np.zeros_like(u)
    np.add.at(routed_out, tok, rows * g[:, None])
    shared_out = np.zeros_like(u)
    for (w1, w3, w2) in shared:
        shared_out += swiglu_ffn(u, w1, w3, w2, hround)
    return u + shared_out + routed_out


def swiglu_backward(x, w1, w3, w2, dy, hround):
    """Matrix form of one expert's backward for rows x [n,d] with output gradient dy
    [n,d] (float64): returns dx [n,d], dW1, dW3 [I,d], dW2 [d,I]; h, da, dv rounded by
    `hround` (the operand type)."""
    a = x @ w1.T
    v = x @ w3.T
    sg = sigmoid(a)
    h = hround(a * sg * v)
    dh = dy @ w2
    da = hround(dh * v * sg * (1.0 + a * (1.0 - sg)))
    dv = hround(dh * a * sg)
    return da @ w1 + dv @ w3, da.T @ x, dv.T @ x, dy.T @ h
