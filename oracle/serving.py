"""Serving outputs of a verification step: which drafted tokens to drop from
the KV cache, and a draft tree's parent array from its list of choices.

TEST INFRASTRUCTURE (see the package header): only tests/, smoke() and the
bench's cpu_baseline leg use it.

* KV-cache trimming: after verification only the KV entries of the accepted
  prefix (chain) or of the accepted root-to-node path (tree) are kept; the
  branches that were rejected are discarded and drafting restarts from the
  confirmed prefix.  (EAGLE-3 review, section on the full inference loop,
  step 5 "KV cache update".)  A serving engine records the dropped tokens in
  a rejected-token mask and replaces their slot-mapping entries with a
  padding slot.  ("[vLLM] EAGLE" code walk, sections on rejected-token
  handling and on slot mapping / KV-cache management.)
* Tree choices: the draft tree is given as a list of tuples, each the child
  ranks along the path from the root to one node, listed level by level (the
  tree depth is the length of the last tuple).  ("[vLLM] EAGLE" code walk,
  section on tree-structured drafting.)

Readings where the pages leave a step open
  - Chain: drafted token i (0-based) of a request is rejected exactly when
    i >= n, n the number of accepted drafts; the emitted correction or bonus
    token is not a draft and has no entry.
  - Tree: node j > 0 is kept exactly when it is the deepest accepted node or
    one of its ancestors; the root (the last confirmed token) is never
    rejected.
  - Choices: choice j is node j + 1 (node 0 the root); its parent is the node
    of the same tuple without its last entry.  A tuple whose parent is not
    listed before it, a tuple listed twice, or a negative rank is an error.
"""
import numpy as np


def rejected_mask_chain(accepted_len, k: int) -> np.ndarray:
    """bool [B, k]: drafted token i of request b is dropped iff i >= n_b."""
    n = np.asarray(accepted_len, dtype=np.int64)
    out = np.zeros((n.shape[0], k), dtype=bool)
    for b in range(n.shape[0]):
        for i in range(k):
            out[b, i] = i >= n[b]
    return out


def kept_nodes(parent, deepest: int) -> set:
    """The deepest accepted node and all its ancestors (root included)."""
    kept = set()
    j = int(deepest)
    while j >= 0:
        kept.add(j)
        j = int(parent[j])
    return kept


def rejected_mask_tree(parent, deepest) -> np.ndarray:
    """bool [B, n_nodes]: node j is dropped iff it is not the deepest
    accepted node of request b nor one of its ancestors."""
    n_nodes = len(parent)
    out = np.zeros((len(deepest), n_nodes), dtype=bool)
    for b, d in enumerate(deepest):
        kept = kept_nodes(parent, d)
        for j in range(n_nodes):
            out[b, j] = j not in kept
    return out


def apply_padding(slot_mapping: np.ndarray, rejected: np.ndarray, pad_slot: int) -> np.ndarray:
    """Slot mapping with every rejected entry replaced by the padding slot."""
    out = np.array(slot_mapping, dtype=np.int64, copy=True)
    out[rejected] = pad_slot
    return out


class TreeChoicesError(ValueError):
    pass


def parent_from_choices(choices) -> list:
    """Parent array (parent[0] = -1) of the tree whose node j + 1 is
    choices[j]."""
    index = {(): 0}
    parent = [-1]
    for j, c in enumerate(choices):
        c = tuple(int(v) for v in c)
        if len(c) < 1 or any(v < 0 for v in c):
            raise TreeChoicesError(f"choice {j} is empty or has a negative rank")
        if c in index:
            raise TreeChoicesError(f"choice {j} is listed twice")
        if c[:-1] not in index:
            raise TreeChoicesError(f"the parent of choice {j} is not listed before it")
        parent.append(index[c[:-1]])
        index[c] = j + 1
    return parent
