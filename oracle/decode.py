"""Decode-time attention over a compressed cache, plain and slow, in numpy float64 (oracle).

TEST INFRASTRUCTURE ONLY: the product path never imports this module.

Source: Krishnan & Schulz, "A JoLT for the KV Cache" (arXiv 2607.12550v2), Sec. 4.5 "Fused decode
kernel": attention of one decode step evaluated over the stored factors and the packed residual,
keys rebuilt and rotated by RoPE before scoring, values taken from the compressed cells, newly
generated tokens held in a small dense tail that shares the softmax.  What that computes is plain
attention over the decoded cache, written out here by definition: decode every cell (Sec. 3,
backbone plus de-rotated residual), apply RoPE to the keys at their positions, softmax of the scaled
scores, weighted sum of the values.

Readings of points the pages leave open (each is listed in the design notes):
  * the cache holds keys before RoPE; a key at token position t is rotated at position t, the tail's
    i-th key at position T + i.  The query arrives already rotated at its own position.
  * RoPE pairs dimension i with i + d_h/2 (the rotate-half layout); the inverse frequencies are the
    fp32 roundings of base^(-2i/d_h), the angle of position t is the fp32 product of fp32(t) and the
    inverse frequency (the fp32 arithmetic of the common implementations), its cosine and sine are
    exact (fp64 here).
  * grouped-query attention: query head j reads KV head j // (n_q / n_h); scores are scaled by
    1 / sqrt(d_h); no mask (one decode step attends to every cached token).
"""
import numpy as np

from . import jolt

__all__ = ["rope_inv_freq", "rope_angles", "apply_rope", "decode_attention", "layer_from_blob"]


def rope_inv_freq(D, base):
    """Inverse frequencies of the D/2 rotation pairs: fp32(base^(-2i/D)), i = 0 .. D/2 - 1."""
    i = np.arange(D // 2, dtype=np.float64)
    return (np.float64(base) ** (-2.0 * i / D)).astype(np.float32)


def rope_angles(positions, inv_freq):
    """[n, D/2] angles: the fp32 product of fp32(position) and each inverse frequency."""
    t = np.asarray(positions, dtype=np.float32)[:, None]
    return (t * inv_freq[None, :].astype(np.float32)).astype(np.float32)


def apply_rope(x, positions, inv_freq):
    """Rotate each row of x [..., n, D] by its position: for i < D/2 the pair (x_i, x_{i+D/2}) turns by
    the angle of (position, i); cosine and sine in fp64 of the fp32 angle."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    a = rope_angles(positions, inv_freq).astype(np.float64)
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def decode_attention(q, K, V, k_tail, v_tail, inv_freq):
    """One decode step of one layer.

    q       [n_q, D]     queries, already rotated at their position.
    K, V    [n_h, T, D]  decoded cache of the layer (keys before RoPE).
    k_tail, v_tail [n_h, n, D] dense tail (keys before RoPE, positions T .. T + n - 1), n may be 0.
    Returns [n_q, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n_q, D = q.shape
    n_h, T, _ = K.shape
    if k_tail is not None and k_tail.shape[1] > 0:
        K = np.concatenate([K, np.asarray(k_tail, dtype=np.float64)], axis=1)
        V = np.concatenate([V, np.asarray(v_tail, dtype=np.float64)], axis=1)
    pos = np.arange(K.shape[1])
    Kr = apply_rope(K, pos, inv_freq)
    g = n_q // n_h
    out = np.empty((n_q, D))
    for j in range(n_q):
        h = j // g
        s = Kr[h] @ q[j] / np.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        out[j] = p @ V[h]
    return out


def layer_from_blob(blob, offsets, dtype, rot_seed, D, n_groups, group_start, seq, layer):
    """Decoded keys and values [n_h, T, D] of one layer of one sequence, from a blob whose cell
    sections are in cell order (sequence, group, K|V)."""
    g = int(np.searchsorted(np.asarray(group_start), layer, side="right") - 1)
    Qrot = jolt.rotation(D, rot_seed)
    out = []
    for t in (0, 1):
        cell = jolt.read_blob_cell(blob, offsets[2 * (seq * n_groups + g) + t], dtype)
        sh = cell["shape"]
        X = jolt.decode_cell(cell["UT"], cell["Ud"], cell["core"], cell["b"], cell["u"], cell["scales"], Qrot,
                             (sh.G, sh.H, sh.T, sh.D))
        out.append(X[layer - group_start[g]])
    return out[0], out[1]
