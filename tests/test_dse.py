"""Host logic of the design-space-exploration drivers against the plain
reference (oracle/dse.py), with synthetic evaluators: identical descent
trajectories and tuning results, identical naive / load-balance / greedy
schedules, DFS optima equal, and the same simulator inputs for a schedule.
The GPU-scored runs are in test_gpu_parity.py."""

import numpy as np
import pytest

from experiment_network_simulation_amd import dse as P
from experiment_network_simulation_amd import inputs as I
from oracle import dse as D

PKT = I.PKT_BYTES


def fake_ticks(algo, nc, chunk, seed):
    """A deterministic rugged landscape standing in for simulated ticks."""
    return (nc * 7919 + (chunk // 32768) * 104729 + algo * 1299709 + seed * 31) % 997 + 1


def run_descent(sizes, start, f):
    d = P.Descent(sizes, start)
    while d.want is not None:
        d.feed(f(d.want))
    return d


def test_descent_state_machine_equals_reference():
    rng = np.random.default_rng(4)
    for trial in range(300):
        M = int(rng.integers(1, 4))
        sizes = tuple(int(x) for x in rng.integers(2, 17, M))
        vals = rng.integers(1, 200, size=sizes)
        f = lambda p: int(vals[p])
        start = tuple(int(rng.integers(0, n)) for n in sizes)
        d = run_descent(sizes, start, f)
        r = D.coordinate_descent(f, sizes, start)
        assert d.trace == r["probes"] and d.best == r["best"] and d.best_t == r["ticks"], trial


def test_lockstep_tuning_equals_sequential_reference():
    tasks = I.tune_tasks_c2(7)
    tasks[3].kind = I.COLL_RING_AG                 # one task with a single subspace
    starts = I.tune_starts(99, len(tasks))
    calls = []

    def evaluate(probes):
        calls.append(len(probes))
        out = []
        for p in probes:
            c = p.work.colls[0]
            out.append(fake_ticks(c.kind, c.nc, c.chunk_bytes, p.ecmp_seed))
        return np.array(out)

    got = P.tune(tasks, starts, evaluate)
    n_probes = 0
    for t, task in enumerate(tasks):
        subs = D.subspaces_of(task.kind)
        profiles = [(lambda a: (lambda q: fake_ticks(a, I.TUNE_NC[q[0]], I.TUNE_CHUNK[q[1]], task.ecmp_seed)))(a)
                    for a in subs]
        ref = D.subspace_tuning(profiles, (16, 16), [starts[t, k] for k in range(len(subs))])
        assert got[t].algo == subs[ref["subspace"]]
        assert (got[t].nc, got[t].chunk) == (I.TUNE_NC[ref["best"][0]], I.TUNE_CHUNK[ref["best"][1]])
        assert got[t].ticks == ref["ticks"]
        for k, run in enumerate(ref["runs"]):
            assert got[t].per_subspace[k]["trace"] == run["probes"]
            n_probes += len(run["profiled"])
    # every distinct point simulated exactly once; each search needs one new
    # point per step, so the steps are as many as the longest search's points
    assert sum(calls) == n_probes
    assert len(calls) == max(len({p for p, _ in s["trace"]}) for r in got for s in r.per_subspace)


def random_tasks(rng, n, a=4, b=6, max_h=3, max_r=3, pk=(1, 2, 4, 8)):
    out = []
    for _ in range(n):
        h = sorted(rng.choice(a, int(rng.integers(1, max_h + 1)), replace=False).tolist())
        r = (10 + rng.choice(b, int(rng.integers(1, max_r + 1)), replace=False)).tolist()
        out.append(I.UnitComm(h, r, int(pk[rng.integers(0, len(pk))]) * PKT))
    return out


def test_schedulers_equal_reference():
    rng = np.random.default_rng(17)
    for trial in range(60):
        tasks = random_tasks(rng, int(rng.integers(1, 12)))
        K = int(rng.choice([1, 2, 4]))
        dur = P.durations(tasks, K)
        assert dur == [D.bcast_duration(u, K) for u in tasks]
        keys = I.greedy_keys(trial, len(tasks), 5)
        for mine, ref in ((P.sched_naive(tasks, dur), D.naive(tasks, dur)),
                          (P.sched_load_balance(tasks, dur), D.load_balance(tasks, dur)),
                          (P.sched_greedy(tasks, dur, keys), D.greedy(tasks, dur, keys))):
            assert mine.sender == ref["sender"] and mine.order == ref["order"], trial
            assert mine.makespan == ref["makespan"]
            assert D.list_schedule(tasks, dur, mine.sender, mine.order)[1] == mine.makespan


def test_dfs_optimum_equals_reference():
    rng = np.random.default_rng(23)
    for trial in range(30):
        tasks = random_tasks(rng, int(rng.integers(1, 6)), a=3, b=4, max_h=2, max_r=2, pk=(1, 2, 3, 5))
        dur = P.durations(tasks, 1)
        mine = P.sched_dfs(tasks, dur)
        ref = D.dfs(tasks, dur)
        assert mine.complete and mine.makespan == ref["makespan"], trial
        assert sorted(mine.order) == list(range(len(tasks)))
        assert all(mine.sender[i] in tasks[i].holders for i in range(len(tasks)))
        assert D.list_schedule(tasks, dur, mine.sender, mine.order)[1] == mine.makespan
        # seeding with an upper bound changes nothing but the work done
        up = P.sched_naive(tasks, dur)
        assert P.sched_dfs(tasks, dur, upper=up).makespan == ref["makespan"]


def test_dfs_budget_reports_incomplete():
    rng = np.random.default_rng(5)
    tasks = random_tasks(rng, 12)
    dur = P.durations(tasks, 1)
    r = P.sched_dfs(tasks, dur, node_budget=50)
    assert not r.complete


def test_schedule_workload_equals_reference():
    rng = np.random.default_rng(31)
    for trial in range(20):
        tasks = random_tasks(rng, int(rng.integers(1, 9)))
        dur = P.durations(tasks, 2)
        s = P.sched_greedy(tasks, dur, I.greedy_keys(trial, len(tasks), 3))
        mine = P.schedule_workload(tasks, s, 2)
        ref = D.schedule_workload(tasks, s.sender, s.order, 2)
        assert [(c.kind, c.nbytes, c.members, c.k) for c in mine.colls] == \
               [(c.kind, c.nbytes, c.members, c.k) for c in ref.colls]
        assert [(t.kind, t.coll, t.preds) for t in mine.tasks] == [(t.kind, t.coll, t.preds) for t in ref.tasks]


def test_invalid_unit_tasks_are_rejected():
    for bad in (I.UnitComm([0], [0, 1], PKT), I.UnitComm([0], [1, 1], PKT), I.UnitComm([], [1], PKT),
                I.UnitComm([0], [], PKT)):
        with pytest.raises(ValueError):
            P.durations([bad], 1)


def test_reshard_scores_every_schedule_in_one_batch():
    rng = np.random.default_rng(2)
    topo = I.single_switch(16)
    inst = [(topo, random_tasks(rng, 5)), (topo, random_tasks(rng, 3))]
    seen = []

    def evaluate(probes):
        seen.append(len(probes))
        return np.array([sum(c.nbytes for c in p.work.colls) // PKT + len(p.work.tasks) for p in probes])

    keys = [I.greedy_keys(s, 5, 2) for s in range(3)]
    out = P.reshard(inst, 2, keys, evaluate, dfs_max_tasks=4)
    assert seen == [2 * (2 + 3) + 1]                 # DFS only for the 3-task instance
    assert out[0].names == ["naive", "load_balance", "greedy0", "greedy1", "greedy2"]
    assert out[1].names[-1] == "dfs"
    assert all(r.best == int(np.argmin(r.simulated)) for r in out)
