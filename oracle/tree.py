"""fp64 numpy rendering of split-KV tree decoding, for checking merge rules.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This follows the steps of "Tree Attention Decoding" (tree_attn_decode.py gist),
function ``tree_attn_decode``, in its order and notation, with the ranks of that
function replaced by a chunk index:

1. scale the query by d^(-1/2);
2. split the keys and values into contiguous chunks the way ``torch.chunk`` does
   (chunk length ceil(L / n), the last one shorter, trailing chunks possibly empty);
3. per chunk: local scores, ``local_max``, ``lse`` of the shifted scores, the local
   softmax times V (``out``), ``den = exp(lse)``, ``num = out * den``;
4. global max over the chunks, renormalise each chunk's ``den`` and ``num`` by
   ``exp(local_max - global_max)``;
5. sum ``den`` and ``num`` over the chunks and divide.

Readings where the gist is silent:
- an empty chunk (the gist would fail on it) is the identity of the merge:
  local_max = -inf, den = 0, num = 0;
- an optional additive bias (ALiBi, see ``oracle_alibi_bias`` in decode_f64.c) is
  added to the scaled scores before the local max;
- steps 4-5 may be applied pairwise in any tree shape.  The pairwise rule is the
  "softmax fusion" formula of "Flash Aandacht: Revolutie in Transformer Efficientie"
  (section on the mathematics), read with un-normalised parts:
  (m1, l1, o1) + (m2, l2, o2) = (m, l1 e^(m1-m) + l2 e^(m2-m), o1 e^(m1-m) + o2 e^(m2-m)),
  m = max(m1, m2); which is steps 4-5 restricted to two chunks.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

Partial = Tuple[float, float, np.ndarray]   # (local_max, den, num)


def chunk_bounds(L: int, n_chunks: int, chunk_len: Optional[int] = None) -> List[Tuple[int, int]]:
    """[lo, hi) of each of n_chunks chunks; empty ones are (lo, lo).

    By default torch.chunk style (length ceil(L / n_chunks)).  ``chunk_len`` fixes the
    length instead -- the reading used when the rows of a batch with different lengths
    share one chunk length (a row then ends with empty chunks)."""
    if L <= 0:
        return [(0, 0)] * n_chunks
    c = chunk_len if chunk_len is not None else -(-L // n_chunks)
    out = []
    for r in range(n_chunks):
        lo = min(r * c, L)
        hi = min(lo + c, L)
        out.append((lo, hi))
    return out


def chunk_partials(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_chunks: int,
                   bias: Optional[np.ndarray] = None, chunk_len: Optional[int] = None) -> List[Partial]:
    """Per-chunk (local_max, den, num) for one query row.

    q [d], k [L, d], v [L, d] (any float dtype; computed in fp64), bias [L] or None;
    chunk_len as in ``chunk_bounds``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    scale = d ** -0.5
    q = q * scale
    parts: List[Partial] = []
    for lo, hi in chunk_bounds(k.shape[0], n_chunks, chunk_len):
        if hi <= lo:
            parts.append((-math.inf, 0.0, np.zeros(v.shape[-1])))
            continue
        sim = k[lo:hi] @ q
        if bias is not None:
            sim = sim + np.asarray(bias[lo:hi], dtype=np.float64)
        local_max = float(sim.max())
        sim = sim - local_max
        lse = math.log(float(np.exp(sim).sum()))
        attn = np.exp(sim - lse)
        out = attn @ v[lo:hi]
        den = math.exp(lse)
        num = out * den
        parts.append((local_max, den, num))
    return parts


def merge_all(parts: Sequence[Partial], order: Optional[Sequence[int]] = None) -> np.ndarray:
    """Steps 4-5: global max, renormalise, sum in the given order, divide."""
    if order is None:
        order = range(len(parts))
    global_max = max(p[0] for p in parts)
    if global_max == -math.inf:
        return np.zeros_like(parts[0][2])
    den = 0.0
    num = np.zeros_like(parts[0][2])
    for i in order:
        local_max, d_i, n_i = parts[i]
        renorm = math.exp(local_max - global_max)
        den = den + d_i * renorm
        num = num + n_i * renorm
    return num / den


def fuse(a: Partial, b: Partial) -> Partial:
    """Pairwise merge of two un-normalised partials (softmax fusion rule)."""
    m = max(a[0], b[0])
    if m == -math.inf:
        return (m, 0.0, a[2] + b[2])
    wa = math.exp(a[0] - m)
    wb = math.exp(b[0] - m)
    return (m, a[1] * wa + b[1] * wb, a[2] * wa + b[2] * wb)


def merge_tree(parts: Sequence[Partial], arity_order: Optional[Sequence[int]] = None) -> np.ndarray:
    """Pairwise (binary tree) merge, leaves taken in ``arity_order``; then divide."""
    level = [parts[i] for i in (arity_order if arity_order is not None else range(len(parts)))]
    while len(level) > 1:
        nxt = [fuse(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    m, l, o = level[0]
    if l == 0.0:
        return np.zeros_like(o)
    return o / l


def tree_decode_row(q, k, v, n_chunks: int, bias=None, chunk_len: Optional[int] = None) -> np.ndarray:
    """The whole tree decode for one query row (steps 1-5)."""
    return merge_all(chunk_partials(q, k, v, n_chunks, bias, chunk_len))
