"""Fixed candidate-tree topologies, built from each head's top-k width.

Medusa heads versus separate draft model ("Trees" paragraph): the step takes
the few best candidates of every head and verifies a tree of their
combinations. The pages fix no rule for which combinations make the tree, so
this module uses a fixed product order:

* a candidate is a path (c_1, ..., c_j), 1 <= j <= K, with c_i < k_i the rank
  chosen from head i's list;
* its score is prod_i 1 / (c_i + 1), so a path never scores above its prefix;
* candidates are sorted by (score descending, depth ascending, path
  lexicographic ascending) and the first N - 1 are kept, plus the root.

The kept set is prefix-closed. Nodes are numbered breadth-first (depth, then
lexicographic), so every parent precedes its children. A topology is given
to the library and to the oracle as two arrays: parent (root: -1) and rank
(the list position the node takes; root: 0). Everything else (depths,
ancestor sets, masks) each side derives on its own.
"""
from __future__ import annotations

from dataclasses import dataclass
from itertools import product
from typing import List, Sequence, Tuple

MAX_NODES = 64


@dataclass(frozen=True)
class Topology:
    paths: Tuple[Tuple[int, ...], ...]  # node i's path of ranks; root = ()
    parent: Tuple[int, ...]
    rank: Tuple[int, ...]

    @property
    def n(self) -> int:
        return len(self.parent)

    def depth_of(self, i: int) -> int:
        return len(self.paths[i])

    def level_counts(self) -> List[int]:
        D = max(len(p) for p in self.paths)
        return [sum(1 for p in self.paths if len(p) == d) for d in range(D + 1)]


def _score_key(path: Tuple[int, ...]):
    den = 1
    for c in path:
        den *= c + 1
    # score = 1/den: larger score first == smaller den first
    return (den, len(path), path)


def product_order_tree(k_per_head: Sequence[int], n_nodes: int) -> Topology:
    K = len(k_per_head)
    if not (1 <= n_nodes <= MAX_NODES):
        raise ValueError("tree must have 1..%d nodes" % MAX_NODES)
    cands = []
    for j in range(1, K + 1):
        for path in product(*[range(k) for k in k_per_head[:j]]):
            cands.append(tuple(path))
    if n_nodes - 1 > len(cands):
        raise ValueError("only %d candidate paths for %d nodes" % (len(cands), n_nodes))
    cands.sort(key=_score_key)
    kept = [()] + cands[: n_nodes - 1]
    kept.sort(key=lambda p: (len(p), p))
    index = {p: i for i, p in enumerate(kept)}
    parent = tuple(-1 if len(p) == 0 else index[p[:-1]] for p in kept)
    rank = tuple(0 if len(p) == 0 else p[-1] for p in kept)
    return Topology(paths=tuple(kept), parent=parent, rank=rank)


def chain(K: int) -> Topology:
    """The top-1 chain: every head contributes only its best candidate."""
    return product_order_tree([1] * K, K + 1)
