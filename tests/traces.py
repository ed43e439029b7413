"""Random call traces for the block pool (alloc / fork / append / truncate / free).

A trace is a list of tuples; ``replay`` drives any object with the pool
methods and records the outcome code of each call, so the oracle's model and
the library's host allocator can be run over the same trace and compared.
"""
from __future__ import annotations

import numpy as np


def random_trace(seed: int, n_ops: int = 60, max_seqs: int = 8, max_tok: int = 40,
                 max_len: int = 160):
    r = np.random.default_rng(seed)
    ops = []
    live = {}
    for _ in range(n_ops):
        kind = r.choice(["alloc", "fork", "append", "append_multi", "truncate", "free"],
                        p=[0.12, 0.14, 0.34, 0.16, 0.16, 0.08])
        free_ids = [s for s in range(max_seqs) if s not in live]
        if kind == "alloc" and free_ids:
            s = int(r.choice(free_ids))
            ops.append(("alloc", s, -1, 0))
            live[s] = 0
        elif kind == "fork" and free_ids and live:
            s = int(r.choice(free_ids))
            p = int(r.choice(list(live)))
            shared = int(r.integers(0, live[p] + 1))
            ops.append(("alloc", s, p, shared))
            live[s] = shared
        elif kind == "append" and live:
            s = int(r.choice(list(live)))
            n = int(r.integers(0, max_tok))
            n = max(0, min(n, max_len - live[s]))
            ops.append(("append", [s], [n]))
        elif kind == "append_multi" and live:
            k = int(r.integers(1, len(live) + 1))
            ss = [int(x) for x in r.choice(list(live), size=k, replace=False)]
            ns = [max(0, min(int(r.integers(0, 6)), max_len - live[s])) for s in ss]
            ops.append(("append", ss, ns))
        elif kind == "truncate" and live:
            s = int(r.choice(list(live)))
            nl = int(r.integers(0, live[s] + 1))
            ops.append(("truncate", s, nl))
        elif kind == "free" and live:
            s = int(r.choice(list(live)))
            ops.append(("free", s))
        # keep our length view in step only for calls that cannot fail on lengths;
        # appends may fail for lack of blocks, so lengths are re-read on replay
        if ops and ops[-1][0] == "append":
            for s, n in zip(ops[-1][1], ops[-1][2]):
                live[s] = live[s] + n
        elif ops and ops[-1][0] == "truncate":
            live[ops[-1][1]] = ops[-1][2]
        elif ops and ops[-1][0] == "free":
            live.pop(ops[-1][1], None)
    return ops
