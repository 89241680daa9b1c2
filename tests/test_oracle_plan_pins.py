"""Pins of the oracle's plan functions against hand-written tables.

``tests/golden/plan_tables.txt`` holds, for each case, the rows worked out by
hand from the definitions (a segment is the token range between two
boundaries, cut into 64-token chunks; a request's pairs are applied in prompt
order; xix.ai HYPIC article, paragraph on linear layers).  The planted
mistakes below (last chunk's tail as length mod 64, chunks rounded down,
step counted from the call's first entry, start taken from the next
boundary, requests shifted by one) must each break at least one table.
"""
import inspect
import os

import numpy as np
import pytest

import oracle

_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_tables.txt")


def _cases():
    cases, cur = [], None
    with open(_GOLDEN) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith(("build ", "compose ")):
                kind, name = line.split(None, 1)
                cur = {"kind": kind, "name": name, "offsets": None, "idx": [], "rows": []}
                cases.append(cur)
                continue
            key, _, val = line.partition(":")
            nums = [int(x) for x in val.split()]
            if key == "offsets":
                cur["offsets"] = nums
            elif key == "idx":
                cur["idx"] = nums
            elif key == "row":
                cur["rows"].append(nums)
            else:
                raise ValueError(f"bad line in {_GOLDEN}: {raw!r}")
    return cases


CASES = _cases()


def _check(plan_build, plan_compose, case):
    if case["kind"] == "build":
        got = plan_build(case["offsets"])
        want = np.array(case["rows"], dtype=np.int64).reshape(-1, 5)
    else:
        got = plan_compose(case["offsets"], case["idx"])
        want = np.array(case["rows"], dtype=np.int64).reshape(-1, 3)
    return got.shape == want.shape and np.array_equal(got, want)


def test_golden_file_covers_the_edge_cases():
    names = {c["name"] for c in CASES}
    for need in ("tails_63_64_65", "empty_segments", "equal_lengths", "empty_chains",
                 "steps_from_each_request", "one_full_chunk"):
        assert need in names
    assert sum(c["kind"] == "build" for c in CASES) >= 6
    assert sum(c["kind"] == "compose" for c in CASES) >= 3


@pytest.mark.parametrize("case", CASES, ids=[c["kind"] + ":" + c["name"] for c in CASES])
def test_plan_matches_hand_table(case):
    assert _check(oracle.plan_build, oracle.plan_compose, case), case["name"]


PLAN_MUTANTS = [
    ("tail as length mod 64 (0 for a full last chunk)",
     "tail = length - CHUNK * (n_chunks - 1) if n_chunks else 0",
     "tail = length % CHUNK"),
    ("chunks rounded down",
     "n_chunks = (length + CHUNK - 1) // CHUNK",
     "n_chunks = length // CHUNK"),
    ("start taken from the next boundary",
     "rows.append((s, off[s], length, n_chunks, tail))",
     "rows.append((s, off[s + 1], length, n_chunks, tail))"),
    ("step counted from the call's first entry",
     "rows = [(r, c - off[r], idx[c])",
     "rows = [(r, c, idx[c])"),
    ("requests shifted by one",
     "rows = [(r, c - off[r], idx[c])",
     "rows = [(r + 1, c - off[r], idx[c])"),
    ("pool index of the previous entry",
     "rows = [(r, c - off[r], idx[c])",
     "rows = [(r, c - off[r], idx[c - 1])"),
]


def _mutated(fn, old, new):
    src = inspect.getsource(fn)
    if old not in src:
        return None
    ns = {"np": np, "CHUNK": oracle.CHUNK}
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[fn.__name__]


@pytest.mark.parametrize("name,old,new", PLAN_MUTANTS, ids=[m[0] for m in PLAN_MUTANTS])
def test_plan_mutant_is_caught(name, old, new):
    pb = _mutated(oracle.plan_build, old, new)
    pc = _mutated(oracle.plan_compose, old, new)
    assert (pb is None) != (pc is None), f"mutation site of {name!r} not found exactly once"
    pb = pb or oracle.plan_build
    pc = pc or oracle.plan_compose
    caught = [c["name"] for c in CASES if not _check(pb, pc, c)]
    assert caught, f"mutant {name!r} passes every hand table"
