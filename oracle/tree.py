"""fp64 numpy split-and-merge decoding, for checking merge rules and per-chunk partials.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The method of "Tree Attention Decoding" (tree_attn_decode.py gist, function
``tree_attn_decode``): cut one query row's keys into contiguous chunks, summarise each
chunk by three numbers computed from its own scores alone, then combine the summaries.
Written here from the mathematics of a softmax over a union of disjoint key sets.

For a chunk C with scores s_j = q.k_j / sqrt(d) (+ bias_j):

    peak(C)   = max_{j in C} s_j
    mass(C)   = sum_{j in C} exp(s_j - peak(C))
    vsum(C)   = sum_{j in C} exp(s_j - peak(C)) v_j              (a vector of width d)

(the gist's local max, denominator and numerator).  Since exp(s_j - P) =
exp(s_j - peak(C)) exp(peak(C) - P) for any reference P, the softmax over all keys is

    out = sum_C exp(peak(C) - P) vsum(C) / sum_C exp(peak(C) - P) mass(C),

with P = max_C peak(C) keeping every factor <= 1 (the gist's global max, renormalise,
sum and divide).  The same identity applied to two summaries at a time gives the
pairwise rule of ``fuse``, so any tree of pairwise merges reaches the same result.

Readings where the gist is silent:
- chunk boundaries follow ``torch.chunk`` (length ceil(L / n), the last one shorter,
  trailing chunks possibly empty), or a given fixed length (rows of one batch sharing
  one chunk length);
- an empty chunk is the identity of the merge: peak = -inf, mass = 0, vsum = 0 (the
  gist itself would fail on one);
- an optional additive bias (ALiBi, ``oracle_alibi_bias`` in decode_f64.c) is part of
  the score before the peak is taken.
"""
from __future__ import annotations

import math
from typing import List, NamedTuple, Optional, Sequence, Tuple

import numpy as np


class Summary(NamedTuple):
    """One chunk's partial: (peak, mass, vsum) as defined in the module docstring."""
    peak: float
    mass: float
    vsum: np.ndarray


def chunk_bounds(L: int, n_chunks: int, chunk_len: Optional[int] = None) -> List[Tuple[int, int]]:
    """[lo, hi) of each of n_chunks chunks; empty ones are (lo, lo).

    By default torch.chunk style (length ceil(L / n_chunks)).  ``chunk_len`` fixes the
    length instead -- the reading used when the rows of a batch with different lengths
    share one chunk length (a row then ends with empty chunks)."""
    if L <= 0:
        return [(0, 0)] * n_chunks
    width = chunk_len if chunk_len is not None else -(-L // n_chunks)
    bounds = []
    for i in range(n_chunks):
        lo = min(i * width, L)
        bounds.append((lo, min(lo + width, L)))
    return bounds


def summarise(scores: np.ndarray, values: np.ndarray) -> Summary:
    """(peak, mass, vsum) of one chunk from its fp64 scores [n] and value rows [n, d]."""
    if scores.shape[0] == 0:
        return Summary(-math.inf, 0.0, np.zeros(values.shape[-1]))
    peak = float(np.max(scores))
    weights = np.exp(scores - peak)
    return Summary(peak, float(np.sum(weights)), weights @ values)


def chunk_partials(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_chunks: int,
                   bias: Optional[np.ndarray] = None, chunk_len: Optional[int] = None) -> List[Summary]:
    """Per-chunk summaries for one query row.

    q [d], k [L, d], v [L, d] (any float dtype; computed in fp64), bias [L] or None;
    chunk_len as in ``chunk_bounds``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    scores = k @ q / math.sqrt(q.shape[-1])
    if bias is not None:
        scores = scores + np.asarray(bias, dtype=np.float64)
    return [summarise(scores[lo:hi], v[lo:hi]) for lo, hi in chunk_bounds(k.shape[0], n_chunks, chunk_len)]


def merge_all(parts: Sequence[Summary], order: Optional[Sequence[int]] = None) -> np.ndarray:
    """All summaries at once, added in ``order``: reference = the largest peak, each
    summary scaled by exp(peak - reference), value sums over mass sums."""
    picks = list(range(len(parts)) if order is None else order)
    ref = max(p.peak for p in parts)
    if ref == -math.inf:                       # every chunk empty: no keys at all
        return np.zeros_like(parts[0].vsum)
    total_mass = 0.0
    total_vsum = np.zeros_like(parts[0].vsum)
    for i in picks:
        scale = math.exp(parts[i].peak - ref)
        total_mass += scale * parts[i].mass
        total_vsum = total_vsum + scale * parts[i].vsum
    return total_vsum / total_mass


def fuse(a: Summary, b: Summary) -> Summary:
    """The summary of the union of two disjoint chunks, from theirs alone."""
    top = max(a.peak, b.peak)
    if top == -math.inf:
        return Summary(top, 0.0, a.vsum + b.vsum)
    sa, sb = math.exp(a.peak - top), math.exp(b.peak - top)
    return Summary(top, sa * a.mass + sb * b.mass, sa * a.vsum + sb * b.vsum)


def merge_tree(parts: Sequence[Summary], leaf_order: Optional[Sequence[int]] = None) -> np.ndarray:
    """Pairwise (binary tree) merge of the summaries taken in ``leaf_order``; then divide."""
    level = [parts[i] for i in (range(len(parts)) if leaf_order is None else leaf_order)]
    while len(level) > 1:
        paired = [fuse(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            paired.append(level[-1])
        level = paired
    root = level[0]
    return np.zeros_like(root.vsum) if root.mass == 0.0 else root.vsum / root.mass


def tree_decode_row(q, k, v, n_chunks: int, bias=None, chunk_len: Optional[int] = None) -> np.ndarray:
    """Chunk, summarise, merge: the whole split decode of one query row."""
    return merge_all(chunk_partials(q, k, v, n_chunks, bias, chunk_len))
