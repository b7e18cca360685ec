"""Paged KV addressing, per-request draft lengths and the verify batch's index
bookkeeping.  TEST INFRASTRUCTURE ONLY (see oracle/__init__).

Sources (page title, section):
  * "Speculative Decoding (EAGLE3) in the vLLM Neuron Framework", The propose()
    Method (a position's cache slot comes from the sequence's block table: the
    block holding pos // block_size, at offset pos % block_size), Design
    Choices (near the length limit a sequence stops speculating and decodes
    one token at a time) and SpecDecodeMetadata: Index Bookkeeping (per
    request, the logits of its draft positions and of one bonus position are
    computed; the index arrays that pick them out of the flat batch).

Readings (the pages leave these open):
  * A request with n draft tokens verifies a prefix of its draft: the first n
    tree nodes in node order (root first, then by depth), which is closed
    under ancestors because every parent precedes its children; for a chain,
    the first n drafts.  n = 0 is plain decoding: the root row alone.
  * In chain mode the final (residual or bonus) draw keeps its own uniform,
    the last one of the request's row, whatever n is.
"""
from __future__ import annotations

import numpy as np

from .tree import Tree


def slot_of(block_table, pos: int, block_size: int) -> int:
    """Physical cache slot of logical position ``pos`` of one sequence."""
    return int(block_table[pos // block_size]) * block_size + pos % block_size


def write_paged(pool, block_table, block_size: int, pos0: int, rows):
    """Store rows[j] (one cache row per position) at positions pos0 + j of a
    sequence, in a pool of shape [n_blocks * block_size, ...]."""
    for j, r in enumerate(rows):
        pool[slot_of(block_table, pos0 + j, block_size)] = r


def gather_paged(pool, block_table, block_size: int, n: int):
    """Positions 0 .. n-1 of a sequence, read back through its block table."""
    return np.stack([pool[slot_of(block_table, p, block_size)] for p in range(n)]) if n else pool[:0]


def spec_decode_metadata(cu_num_scheduled_tokens, num_draft_tokens, input_ids=None):
    """Index arrays of one verify batch.

    Request b owns the flat input positions [cu[b-1], cu[b]) (cu[-1] = 0); its
    last num_draft_tokens[b] tokens are drafts.  The target's logits are needed
    at the nd + 1 positions that end the request (each draft is checked against
    the logits of the position before it, and the last position gives the
    bonus).  Returns a dict:
      cu_num_draft_tokens    running total of draft tokens;
      logits_indices         the flat positions whose logits are computed,
                             request by request;
      target_logits_indices  which entries of logits_indices verify a draft;
      bonus_logits_indices   which entry of logits_indices is each request's
                             bonus position (its last);
      draft_token_ids        input_ids at the draft positions (when given).
    """
    cu = [int(x) for x in cu_num_scheduled_tokens]
    nd = [int(x) for x in num_draft_tokens]
    out = {"cu_num_draft_tokens": [], "logits_indices": [], "target_logits_indices": [],
           "bonus_logits_indices": [], "draft_token_ids": []}
    total = 0
    for b in range(len(cu)):
        start = cu[b - 1] if b > 0 else 0
        assert nd[b] >= 0 and nd[b] + 1 <= cu[b] - start, "a request needs nd + 1 scheduled tokens"
        total += nd[b]
        out["cu_num_draft_tokens"].append(total)
        first = len(out["logits_indices"])
        for t in range(nd[b] + 1):
            out["logits_indices"].append(cu[b] - nd[b] - 1 + t)
        for t in range(nd[b]):
            out["target_logits_indices"].append(first + t)
            if input_ids is not None:
                out["draft_token_ids"].append(int(input_ids[cu[b] - nd[b] + t]))
        out["bonus_logits_indices"].append(first + nd[b])
    return out


def truncate_tree(tree: Tree, n_draft: int) -> Tree:
    """The request's verified draft: its first n_draft nodes (plus the root)."""
    n = max(0, min(int(n_draft), len(tree.tokens) - 1)) + 1
    assert all(p < i for i, p in enumerate(tree.parents[:n]) if i > 0)
    return Tree(list(tree.tokens[:n]), list(tree.parents[:n]), list(tree.depth[:n]), list(tree.score[:n]),
                list(tree.expanded_as[:n]))
