"""Retrieve-and-inject: gather pre-RoPE K/V, rotate K, scatter into a paged cache.

Source: the InferScale review (arXiv 2607.27090): "Referee Report", Summary
(facts stored pre-RoPE, re-rotated with Chunked RoPE, scatter-copied into
vLLM's paged KV cache); "What carries the argument" (re-rotate keys to
serving-time positions on injection); Figure 2 caption (top-k facts resolved
to their KV by fact_id and positioned by chunked RoPE).

Readings:
* Store layout: K and V arenas [L][C][H][D] of bfloat16 bits; fact f owns rows
  [row0_f, row0_f + len_f) in every layer.
* Cache layout: per layer, [num_blocks][block_size][H][D] bfloat16 ("NHD");
  a slot is block * block_size + offset.
* K is rotated in float64 and rounded once to bfloat16 (nearest, ties to
  even); V is copied bit for bit.
* Pre-RoPE store: a key is rotated to its token's serving position.
  Chunk-local store (keys already rotated at positions 0 .. len-1 of their own
  fact, as when a fact is encoded alone): a key is rotated by the fact's
  serving start s, R(s) R(t) = R(s + t) (Theorem 6's axiom R_a^T R_b =
  R_{b-a}); the stored key has already been rounded once, so the two stores
  agree to within that rounding, not bit for bit.
"""

import numpy as np

from . import bf16, paged, rope


def rotate_k_bits(k_bits, pos, base, style=rope.HALF_SPLIT, scaling=None):
    """Rotate bfloat16 keys k_bits[..., D] by positions pos; bf16 bits out."""
    x = bf16.bf16_bits_to_f64(k_bits)
    return bf16.f64_to_bf16_bits(rope.rotate(x, pos, base, style=style, scaling=scaling))


class PagedImage:
    """Host image of some physical blocks of a per-layer paged cache (K or V).

    data: uint16 [L][n_listed][block_size][H][D]; block_ids[i] names data[:, i].
    """

    def __init__(self, num_layers, block_ids, block_size, num_heads, head_dim, fill):
        self.block_ids = [int(b) for b in block_ids]
        self.index = {b: i for i, b in enumerate(self.block_ids)}
        if len(self.index) != len(self.block_ids):
            raise ValueError("block ids must be distinct")
        self.block_size = int(block_size)
        self.data = np.full(
            (num_layers, len(self.block_ids), block_size, num_heads, head_dim),
            np.uint16(fill), dtype=np.uint16)

    def row(self, layer, slot):
        """View of one slot's [H][D] row in one layer."""
        b, off = divmod(int(slot), self.block_size)
        return self.data[layer, self.index[b], off]


def inject(k_arena, v_arena, fact_rows, requests, block_size, base, k_image, v_image,
           style=rope.HALF_SPLIT, scaling=None, chunk_local=False):
    """Naive per-token scatter of rotated K and copied V into k_image / v_image.

    k_arena, v_arena: indexable as [layer][row] -> [H][D] uint16 bf16 bits.
    fact_rows: fact_id -> (first row, length).  requests: (fact_ids, prefix, block_table).
    style, scaling: RoPE pairing and frequency rule (oracle.rope).
    chunk_local: the arena holds keys rotated at chunk-local positions.
    Returns the number of tokens injected.
    """
    src_row, pos, slot = paged.token_mapping(requests, fact_rows, block_size)
    angle = paged.rotation_positions(requests, fact_rows, chunk_local)
    num_layers = k_image.data.shape[0]
    for r, a, s in zip(src_row, angle, slot):
        for layer in range(num_layers):
            k_image.row(layer, s)[...] = rotate_k_bits(k_arena[layer][r], a, base, style,
                                                       scaling)
            v_image.row(layer, s)[...] = v_arena[layer][r]
    return len(src_row)
