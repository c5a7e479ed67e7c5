"""Oracle O4: decode attention by its plain definition, in float64 (test infrastructure only).

What it follows:

* PagedAttention blog, "The Attention Kernel": scores are the query against
  every key of the sequence, divided by the square root of the head dimension,
  softmax-normalised, and used to weight the values.  The blog's kernel walks
  the block table block by block with an online softmax and merges partial
  results across thread blocks with a log-sum-exp step; in exact arithmetic
  both give the plain softmax, so the oracle does not split and uses the
  two-pass form (max, then normalised weights).
* PageFault, "Four stages" (stages 1 and 3): paged attention has the same math
  as contiguous attention; only the K/V loads go through the block table.  Here
  that is literal: the paged oracle reads K/V back through the tables
  (``layout.readback``) and then calls the contiguous definition.

Readings where the pages are silent:

* Only positions below the context length are tokens (PageFault, "Design
  notes": the last page's unused tail); they are never read.
* The decode query attends to every cached token including the one written this
  step; no causal mask beyond the length.
* A sequence of length 0 yields a zero output.
* Grouped-query attention (not on the pages): query head h reads kv head
  ``h // (Hq // Hkv)``.
* Stored 16-bit and 32-bit values are decoded exactly to float64 first.
"""
import math

import numpy as np

from . import layout


def decode_bits(bits, dtype):
    """Exact float64 value of stored bit patterns of ``dtype`` ('f32', 'f16', 'bf16')."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # bfloat16 is the top half of a binary32 word.
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def attention(q, K, V, scale):
    """softmax(scale * K q) weighted sum of V rows, for one query vector.

    ``q`` is ``[D]``, ``K`` and ``V`` are ``[n][D]`` float64.  Returns ``[D]``.
    """
    n = K.shape[0]
    if n == 0:
        return np.zeros(q.shape[0], dtype=np.float64)
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def default_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)


def paged_decode_attention(q_bits, pool, g, layer, tables, lengths, dtype, scale=None):
    """Decode attention for every (sequence, query head) through the block tables.

    ``q_bits`` is ``[n][Hq][D]`` stored bits; ``tables[s]`` the block table of
    sequence s and ``lengths[s]`` its context length.  Returns ``[n][Hq][D]``
    float64.
    """
    q = decode_bits(q_bits, dtype)
    n, hq, d = q.shape
    if hq % g.H != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    group = hq // g.H
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((n, hq, d), dtype=np.float64)
    for s in range(n):
        kc, vc = layout.readback(pool, g, layer, tables[s], int(lengths[s]))
        K = decode_bits(kc, dtype)
        V = decode_bits(vc, dtype)
        for h in range(hq):
            hk = h // group
            out[s, h] = attention(q[s, h], K[:, hk, :], V[:, hk, :], scale)
    return out


def contiguous_decode_attention(q, K, V, lengths, scale=None):
    """Same as ``paged_decode_attention`` on already-decoded contiguous float64 K/V.

    ``K[s]``, ``V[s]`` are ``[len_s][Hkv][D]``.
    """
    n, hq, d = q.shape
    hkv = K[0].shape[1] if n else 1
    group = hq // hkv
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((n, hq, d), dtype=np.float64)
    for s in range(n):
        ln = int(lengths[s])
        for h in range(hq):
            out[s, h] = attention(q[s, h], K[s][:ln, h // group, :], V[s][:ln, h // group, :], scale)
    return out


def attention_bruteforce(q, K, V, scale):
    """Pure-Python version used to pin ``attention`` on tiny inputs.

    Each score is a correctly rounded sum (``math.fsum``); the weights use
    ``math.exp`` without any max shift (fine for the small inputs it is used
    on) and the normalisation is a separate division, one output at a time.
    """
    n = len(K)
    d = len(q)
    if n == 0:
        return [0.0] * d
    scores = [scale * math.fsum(float(q[i]) * float(K[j][i]) for i in range(d)) for j in range(n)]
    weights = [math.exp(z) for z in scores]
    total = math.fsum(weights)
    return [math.fsum(weights[j] * float(V[j][i]) for j in range(n)) / total for i in range(d)]
