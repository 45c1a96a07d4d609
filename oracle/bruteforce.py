"""Textbook contiguous attention in fp64 (numpy + scipy), with no block table at all.

TEST INFRASTRUCTURE ONLY. This is the special case the paged method reduces to when a
sequence's K/V rows are stored contiguously in logical order ([P1] "PagedAttention",
inferensys.com: the kernel gathers the rows a contiguous layout would hold; [P2] "Paged
Attention", infra.pidoku.co.in, §5 "The kernel side": the same q·k / softmax / p·v, with
only the address of each block changed). It is written independently of pa_oracle.c and
uses scipy's softmax, so a dropped term, a wrong head mapping or a transposed operand in
either one shows up as a disagreement between the two.
"""
import numpy as np
from scipy.special import softmax


def bf16_bits_to_f64(bits):
    """Raw bf16 bits (uint16) -> float64; exact."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def attention(q, K, V, scale):
    """softmax(scale * q K^T) V for one sequence.

    q [Hq, D]; K, V [L, Hkv, D] in logical token order; query head h uses KV head
    h // (Hq // Hkv). Returns float64 [Hq, D]; an empty sequence gives zeros.
    """
    q = to_f64(q)
    K = to_f64(K)
    V = to_f64(V)
    Hq, D = q.shape
    L, Hkv, _ = K.shape
    group = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if L == 0:
        return out
    s64 = float(np.float32(scale))
    for h in range(Hq):
        g = h // group
        scores = s64 * (K[:, g, :] @ q[h])
        out[h] = softmax(scores) @ V[:, g, :]
    return out


def causal_attention(Q, K, V, scale):
    """Causal softmax attention of a sequence's last n tokens, in matrix form.

    Q [n, Hq, D] are the queries of positions L - n .. L - 1; K, V [L, Hkv, D] in logical
    token order. Query j may see tokens 0 .. L - n + j: the scores above that diagonal are
    set to -inf before the row softmax. Returns float64 [n, Hq, D].
    """
    Q = to_f64(Q)
    K = to_f64(K)
    V = to_f64(V)
    n, Hq, D = Q.shape
    L, Hkv, _ = K.shape
    group = Hq // Hkv
    out = np.zeros((n, Hq, D), dtype=np.float64)
    if n == 0:
        return out
    s64 = float(np.float32(scale))
    visible = np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None]     # [n, L]
    for h in range(Hq):
        g = h // group
        S = s64 * (Q[:, h, :] @ K[:, g, :].T)
        S = np.where(visible, S, -np.inf)
        out[:, h, :] = softmax(S, axis=1) @ V[:, g, :]
    return out
