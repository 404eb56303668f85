"""Exact top-k retrieval by inner product, float64.

Source: the InferScale review (arXiv 2607.27090), "Referee Report", Summary
(facts are retrieved at serving time through a GPU index, then their KV is
injected) and Figure 2 caption (every fact has a retrieval embedding under its
fact_id).  The pages use an approximate index; the review's "Circularity
Check" states the backend changes latency, not the facts found, so the oracle
is the exact definition.

Readings: the score of fact f for query q is the inner product q . e_f of the
bf16 values (exact products, summed in float64); the top k are the k highest
scores, best first, equal scores ordered by smaller fact id.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64


def scores(q_bits, emb_bits):
    """q_bits [E], emb_bits [F][E] (bf16 bits) -> float64 [F] inner products."""
    q = bf16_bits_to_f64(q_bits)
    e = bf16_bits_to_f64(emb_bits)
    return e @ q


def topk(score, k):
    """Indices of the k best scores (higher first, then smaller index)."""
    score = np.asarray(score, dtype=np.float64)
    idx = np.arange(len(score))
    order = np.lexsort((idx, -score))   # primary key -score, then index
    return order[:k]
