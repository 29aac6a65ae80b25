"""Oracle for AllGather-MoE: routing, arrival-ordered row lists, grouped GEMM.

Test infrastructure only.

* DITRON §4.1 (AG-MoE workload): the tokens of all ranks are all-gathered and
  each expert's tokens go through that expert's weight (a grouped GEMM).
* The router is the usual top-k softmax gate: every token picks the k experts
  with the largest logits; its gate weights are a softmax over those k logits.
  Ties between equal logits go to the lower expert index, which makes the
  selection unique.  The gates are an output of routing; they are not applied
  to the grouped-GEMM rows (they belong to the combine after the down
  projection, which is outside this path).
* Device-level chunks have data-dependent sizes computed at run time (DITRON
  §3.1, device-level interface: dynamic shapes for MoE routing).
* Within an expert, rows are ordered by how early their token's chunk arrives
  (consume position, then token index), so that tiles needing only early chunks
  come first (talk, "MoE dynamic sorting").
"""
from __future__ import annotations

import numpy as np

from .gemm import bf16_to_f64


def topk_select(logits_row: np.ndarray, k: int):
    """Indices of the k largest entries, largest first; equal values -> lower index first."""
    order = sorted(range(len(logits_row)), key=lambda e: (-float(logits_row[e]), e))
    return order[:k]


def softmax(vals) -> np.ndarray:
    v = np.asarray(vals, dtype=np.float64)
    e = np.exp(v - v.max())
    return e / e.sum()


def route(logits: np.ndarray, k: int, world: int, rank: int, tokens_per_chunk: int):
    """Routing outputs.

    Returns a dict with
      topk     T x k int32   selected experts, by decreasing logit
      gates    T x k float64 softmax over the selected logits
      counts   E     int32   tokens per expert
      offsets  E+1   int32   exclusive prefix sum of counts
      row_token T*k  int32   source token of every grouped-GEMM row (expert-major;
                             inside an expert ordered by (consume position of the
                             token's chunk, token))
      slot     T x k int32   grouped-GEMM row that holds token t's j-th expert
    """
    T, E = logits.shape
    topk = np.zeros((T, k), np.int32)
    gates = np.zeros((T, k), np.float64)
    for t in range(T):
        sel = topk_select(logits[t], k)
        topk[t] = sel
        gates[t] = softmax([logits[t, e] for e in sel])
    counts = np.zeros(E, np.int32)
    for t in range(T):
        for e in topk[t]:
            counts[e] += 1
    offsets = np.zeros(E + 1, np.int32)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    members = [[] for _ in range(E)]
    for t in range(T):
        for e in topk[t]:
            members[e].append(t)
    row_token = np.zeros(T * k, np.int32)
    slot = np.zeros((T, k), np.int32)
    for e in range(E):
        ordered = sorted(members[e], key=lambda t: (((t // tokens_per_chunk) - rank) % world, t))
        for i, t in enumerate(ordered):
            row_token[offsets[e] + i] = t
    where = {}
    for i, t in enumerate(row_token):
        where[(int(t), int(np.searchsorted(offsets, i, side="right") - 1))] = i
    for t in range(T):
        for j in range(k):
            slot[t, j] = where[(t, int(topk[t, j]))]
    return dict(topk=topk, gates=gates, counts=counts, offsets=offsets, row_token=row_token,
                slot=slot)


def gather_tokens(x_chunks) -> np.ndarray:
    return np.concatenate([bf16_to_f64(x) for x in x_chunks], axis=0)


def grouped_gemm(x_chunks, w: np.ndarray, offsets, row_token, rows=None) -> np.ndarray:
    """Y[i] = X[row_token[i]] @ W_e for the expert e whose segment holds row i.

    ``w`` is E x K x N bf16 bits.  ``rows`` optionally restricts the computation
    to some output rows (sampled checks at full size)."""
    X = gather_tokens(x_chunks)
    E = w.shape[0]
    n_rows = int(offsets[E])
    idx = np.arange(n_rows) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(idx), w.shape[2]), np.float64)
    experts = np.searchsorted(np.asarray(offsets), idx, side="right") - 1
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        toks = np.asarray(row_token)[idx[sel]]
        out[sel] = X[toks] @ bf16_to_f64(w[e])
    return out
