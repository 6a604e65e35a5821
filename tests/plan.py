"""Executes a workload's pool plan with any pool object.

Neutral test helper: imports neither the oracle nor the library.  The pool
must offer ``allocate_sequence(L, bs)``, ``fork(table)`` and ``alloc()``.
"""

from workloads.synth import plan_ops


def build_tables(w, pool):
    tables = [None] * w.S
    for op in plan_ops(w):
        kind, s = op[0], op[1]
        if kind == "new":
            tables[s] = pool.allocate_sequence(op[2], w.BS)
        elif kind == "share":
            tables[s] = pool.fork(tables[op[2]][: op[3]])
        elif kind == "grow":
            while len(tables[s]) * w.BS < op[2]:
                tables[s].append(pool.alloc())
    return tables
