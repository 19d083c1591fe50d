"""Planted mistakes: every pin must be able to fail.

Each case copies oracle/oracle.c, plants one plausible mistake by replacing an
exact piece of its text (a dropped term, a wrong sign or index, a swapped
operand), compiles the copy with gcc into a temporary library, and runs the
pins that should catch it in a fresh pytest process pointed at that library
(MSIM_ORACLE_LIB).  The case passes only if those pins fail.  Nothing here
runs on a GPU, and the committed oracle is never modified.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

PINS = "tests/test_oracle_pins.py"
STEP = "tests/test_oracle_stepper.py"
UNEVEN = [f"{PINS}::test_ring_uneven_chunks_and_fold"]
GRID = [f"{STEP}::test_rings_exhaustive_grid[0]", f"{STEP}::test_rings_exhaustive_grid[3]",
        f"{STEP}::test_rings_exhaustive_grid[5]"]
HAND = [f"{PINS}::test_hand_traces"]

# (name, text in oracle.c, replacement, pins that must catch it)
MUTANTS = [
    ("chunk order (i + s) instead of (i - s)",
     "return (uint32_t)(((int64_t)i - s % N + N) % N);", "return (uint32_t)(((int64_t)i + s % N) % N);",
     UNEVEN),
    ("second all-reduce half one chunk off",
     "return (uint32_t)(((int64_t)i + 1 - s2 + 2 * (int64_t)N) % N);",
     "return (uint32_t)(((int64_t)i - s2 + 2 * (int64_t)N) % N);", UNEVEN),
    ("last round never folded", "if (R > 1 && Pc - (R - 1) * N * p < N) R--;", "",
     UNEVEN + [f"{PINS}::test_fold_flow_count"]),
    ("chunk remainder given to the last chunks", "(k < X % N)", "(k >= N - X % N)", UNEVEN),
    ("channel remainder given to the last channels", "(c < P % NC)", "(c >= NC - P % NC)", UNEVEN + GRID),
    ("digest mixer constant", "0xbf58476d1ce4e5b9ull", "0xbf58476d1ce4e5b7ull",
     [f"{PINS}::test_mix64_is_splitmix64"]),
    ("digest keyed by (RD, flow)", "mix64(((uint64_t)f << 32) | t)", "mix64(((uint64_t)t << 32) | f)",
     [f"{PINS}::test_digest_is_sum_over_flows"]),
    ("switch round-robin pointer not advanced", "pp->rr = (pp->granted + 1) % deg;", "pp->rr = pp->granted;",
     HAND + GRID),
    ("NIC round-robin pointer not advanced", "pp->rr = (pp->granted + 1) % n_in;", "pp->rr = pp->granted;",
     GRID + [f"{STEP}::test_incast_and_all_to_all"]),
    ("credit sees the pops and pushes of earlier rounds of the tick", "pp->credit <= 0) continue;",
     "(x->layer[pp->peer_node] != 0 && (int64_t)x->Q - (int64_t)x->port[pp->peer_port].occ <= 0)) continue;",
     GRID),
    ("packets forwarded before they arrive", "if (head && head->arrive <= t)", "if (head)",
     HAND + [f"{PINS}::test_single_flow_latency"]),
    ("activation one tick late", "if (when == NONE || when > t)", "if (when == NONE || when >= t)",
     UNEVEN + [f"{PINS}::test_c1_nc1_values"]),
    ("send completion without the + 1", "if (fl->sent == fl->size) { fl->sd = t + 1; c->cur++; }",
     "if (fl->sent == fl->size) { fl->sd = t; c->cur++; }", UNEVEN),
]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, pins):
    src = open(SRC).read()
    assert old in src, f"mutation target not found: {old}"
    mutated = src.replace(old, new)
    c_file = tmp_path / "oracle_mutant.c"
    so = tmp_path / "liboracle_mutant.so"
    c_file.write_text(mutated)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-w", "-shared", "-fPIC", str(c_file), "-o", str(so)])
    env = dict(os.environ, MSIM_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    # exit code 1: tests ran and at least one failed (not a collection or usage error)
    assert r.returncode == 1, f"{name}: pins did not catch it\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
