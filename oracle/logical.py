"""The logical (contiguous) view of each sequence: which token rows it holds, in order.

[exp] 「PagedAttention：向操作系统借思路」: the model still sees one contiguous logical sequence;
only the physical blocks are scattered, and the block table restores contiguity on access.
[day28] §三 3.2: paged attention performs the same computation as over contiguous K/V.
This class keeps that contiguous view, with no blocks at all, so that paged results can be
checked against dense attention.
"""
from typing import Dict, List, Sequence, Tuple


class LogicalSeqs:
    def __init__(self):
        self.rows: Dict[int, List[int]] = {}

    def apply(self, op: Tuple) -> None:
        kind = op[0]
        if kind == "add":
            assert op[1] not in self.rows
            self.rows[op[1]] = []
        elif kind == "append":
            _, sid, n, tok0 = op
            self.rows[sid].extend(range(tok0, tok0 + n))
        elif kind == "fork":
            _, parent, child = op
            assert child not in self.rows
            self.rows[child] = list(self.rows[parent])
        elif kind == "free":
            del self.rows[op[1]]
        else:
            raise ValueError(kind)

    def apply_all(self, ops: Sequence[Tuple]) -> None:
        for op in ops:
            self.apply(op)

    def token_rows(self, sid: int, length: int = None) -> List[int]:
        r = self.rows[sid]
        return list(r if length is None else r[:length])
