"""Serving-time positions and paged-cache slots, with plain Python loops.

Source: the InferScale review (arXiv 2607.27090).
* "If this is right", second bullet, and "invented entities: Chunked RoPE":
  facts encoded once are placed at arbitrary prompt positions, in whatever
  order retrieval returns them (dynamic top-k assembly).
* "Axiom & Free-Parameter Ledger", axiom on vLLM's KV-connector (section 3.4):
  a prompt prefix is marked as externally available and paged blocks are
  allocated without prefill; K/V are then scatter-copied into them.
* "Referee Report", Summary: the target is vLLM's paged KV cache
  (PagedAttention, reference [6]).

Readings:
* Positions are 0-based.  The request's prefix occupies [0, P); the retrieved
  facts follow it contiguously in the order of the request's fact-id list.
* A request's block table lists physical block ids; logical position p lives
  in physical slot  block_table[p // block_size] * block_size + p % block_size.
* Only fact tokens are written; prefix and query slots are never touched.
"""


def fact_positions(prefix_len, fact_lengths):
    """Positions of each fact's tokens, facts in list order after the prefix."""
    out = []
    p = int(prefix_len)
    for length in fact_lengths:
        out.append(list(range(p, p + int(length))))
        p += int(length)
    return out


def slot_of(pos, block_table, block_size):
    """Physical slot of logical position pos under a block table."""
    pos = int(pos)
    return int(block_table[pos // block_size]) * block_size + pos % block_size


def token_mapping(requests, fact_rows, block_size):
    """Per injected token: (arena row, position, slot), in request, fact, token order.

    requests: iterable of (fact_ids, prefix_len, block_table).
    fact_rows: mapping fact_id -> (first arena row, length).
    Returns three Python lists of ints.
    """
    src_row, pos_out, slot_out = [], [], []
    for fact_ids, prefix_len, block_table in requests:
        lengths = [fact_rows[int(f)][1] for f in fact_ids]
        for f, positions in zip(fact_ids, fact_positions(prefix_len, lengths)):
            row0 = fact_rows[int(f)][0]
            for t, p in enumerate(positions):
                src_row.append(row0 + t)
                pos_out.append(p)
                slot_out.append(slot_of(p, block_table, block_size))
    return src_row, pos_out, slot_out


def rotation_positions(requests, fact_rows, chunk_local=False):
    """Per injected token (same order as token_mapping): the position its key
    is rotated by.  Pre-RoPE keys: the token's serving position.  Keys stored
    rotated at chunk-local positions 0 .. len-1: the fact's first serving
    position (the relocation offset), the same for every token of the fact."""
    out = []
    for fact_ids, prefix_len, _ in requests:
        lengths = [fact_rows[int(f)][1] for f in fact_ids]
        for positions in fact_positions(prefix_len, lengths):
            for p in positions:
                out.append(positions[0] if chunk_local else p)
    return out
