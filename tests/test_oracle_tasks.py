"""Pins of the oracle's task graph: the System Simulator's schedule of compute
tasks, intra-server collectives (the alpha + size / beta analytical model) and
packet-level collectives.

Expected values come from closed forms that follow from the task rules (a task
starts when its last predecessor has finished; a compute or intra-server task
lasts its duration; a collective task finishes when its last flow arrives) and
from the ring closed form already pinned for the collectives themselves.
"""

import numpy as np
import pytest

from experiment_network_simulation_amd import inputs as I

PKT = I.PKT_BYTES


def ring_ag(N, R, p, L):
    """NC = 1 ring all-gather, every chunk p packets, no contention, latency L."""
    tau = L + p - 1
    return (R - 1) * ((N - 2) * tau + p) + (N - 1) * tau


def run(oracle, w, n_hosts, delay=1, queue=8):
    b = I.single_batch(I.single_switch(n_hosts, 1, delay), w, queue_pkts=queue)
    r = oracle.run(b, 0, check=True, flows=True)
    assert r["rc"] == 0 and r["status"] == oracle.OK
    return r


@pytest.mark.parametrize("d0,d1,N,R,p", [(5, 3, 4, 1, 2), (1, 1, 3, 2, 1), (17, 9, 6, 3, 2), (2, 40, 2, 1, 5)])
def test_compute_collective_chain(oracle, d0, d1, N, R, p):
    """compute(d0) -> ring all-gather -> compute(d1): T = d0 + T_ring + d1."""
    w = I.Workload([I.ring(I.COLL_RING_AG, R * N * p * PKT, range(N), 1, p * PKT)])
    w.tasks = [I.compute(d0), I.comm(0, [0]), I.compute(d1, [1])]
    r = run(oracle, w, N)
    T_ring = ring_ag(N, R, p, 2)
    assert list(r["task_start"]) == [0, d0, d0 + T_ring]
    assert list(r["task_finish"]) == [d0, d0 + T_ring, d0 + T_ring + d1]
    assert r["t_end"] == d0 + T_ring + d1
    # the collective's first flows activate exactly at the task's start
    assert int(r["act"].min()) == d0


@pytest.mark.parametrize("alpha,nbytes,beta", [(3, 1000, 100), (1, 4096, 4096), (7, 1, 1000), (0, 10, 3)])
def test_intra_server_analytical_duration(oracle, alpha, nbytes, beta):
    """An intra-server collective lasts alpha + ceil(bytes / beta) ticks."""
    w = I.Workload()
    w.tasks = [I.intra(alpha, nbytes, beta), I.compute(2, [0])]
    b = I.single_batch(I.single_switch(2), w)
    r = oracle.run(b, 0, flows=True)
    D = alpha + -(-nbytes // beta)
    assert list(r["task_finish"]) == [D, D + 2] and r["t_end"] == D + 2


def test_fork_join_and_overlap(oracle):
    """compute(4) forks two rings on disjoint hosts and an overlapping compute;
    the join starts at the latest of the three."""
    N, p = 3, 2
    w = I.Workload([I.ring(I.COLL_RING_AG, N * p * PKT, [0, 1, 2], 1, p * PKT),
                    I.ring(I.COLL_RING_AG, 2 * N * p * PKT, [3, 4, 5], 1, p * PKT)])
    w.tasks = [I.compute(4), I.comm(0, [0]), I.comm(1, [0]), I.compute(11, [0]), I.compute(5, [1, 2, 3])]
    r = run(oracle, w, 6)
    t1, t2 = 4 + ring_ag(N, 1, p, 2), 4 + ring_ag(N, 2, p, 2)
    assert list(r["task_finish"][:4]) == [4, t1, t2, 15]
    assert r["task_start"][4] == max(t1, t2, 15)
    assert r["t_end"] == max(t1, t2, 15) + 5


def test_untasked_collectives_start_at_zero(oracle):
    """Collectives no task names start at tick 0, alongside the task graph."""
    w = I.Workload([I.ring(I.COLL_RING_AG, 4 * PKT, range(4), 1, PKT),
                    I.ring(I.COLL_RING_AG, 4 * PKT, [4, 5, 6, 7], 1, PKT)])
    w.tasks = [I.compute(30), I.comm(1, [0])]
    r = run(oracle, w, 8)
    assert int(r["act"][:12].min()) == 0           # collective 0: no task
    assert int(r["act"][12:].min()) == 30          # collective 1: after the compute
    assert r["t_end"] == 30 + ring_ag(4, 1, 1, 2)


def test_task_activation_rule_on_a_mixed_graph(oracle):
    """Every task starts exactly at the latest finish of its predecessors, and
    every flow that is first on its connection in a task's collective
    activates no earlier than the task's start (exactly at it when nothing
    else holds it back: the ring's first step)."""
    rng = np.random.default_rng(5)
    topo = I.leaf_spine(2, 4, 2)
    colls, tasks = [], [I.compute(3)]
    for j in range(5):
        hosts = [int(x) for x in rng.permutation(8)[:int(rng.integers(2, 6))]]
        colls.append(I.ring(I.COLL_RING_AR, len(hosts) * 2 * PKT * int(rng.integers(1, 3)), hosts, 1, 2 * PKT))
        tasks.append(I.comm(j, [int(rng.integers(0, len(tasks)))]))
        tasks.append(I.intra(int(rng.integers(1, 5)), int(rng.integers(1, 5000)), 1000, [len(tasks) - 1]))
    w = I.Workload(colls)
    w.tasks = tasks
    b = I.single_batch(topo, w, queue_pkts=8, ecmp_seed=9)
    r = oracle.run(b, 0, check=True, flows=True)
    assert r["status"] == oracle.OK
    for k, tk in enumerate(tasks):
        want = max((int(r["task_finish"][q]) for q in tk.preds), default=0)
        assert int(r["task_start"][k]) == want, k
    f0 = 0
    for j, c in enumerate(colls):
        N = len(c.members)
        S = 2 * (N - 1)
        k = 1 + 2 * j                                 # the collective's task
        first = f0 + np.arange(N)                     # round 0, step 0: the first flow of each connection
        assert np.all(r["act"][first] == r["task_start"][k])
        Pc = c.nbytes // PKT
        R = -(-Pc // (N * 2))
        if R > 1 and Pc - (R - 1) * N * 2 < N:
            R -= 1
        f0 += R * S * N
    assert r["t_end"] == max(int(r["rd"].max()), int(r["task_finish"].max()))


def test_task_validation(oracle):
    topo = I.single_switch(4)
    ring = I.ring(I.COLL_RING_AG, 4 * PKT, range(4), 1, PKT)
    bad = [
        [I.compute(0)],                                  # zero duration
        [I.compute(2, [0])],                             # predecessor not earlier
        [I.comm(1)],                                     # no such collective
        [I.comm(0), I.comm(0)],                          # named twice
        [I.intra(0, 0, 5)],                              # zero duration
        [I.intra(1, 10, 0)],                             # zero bandwidth
    ]
    for tasks in bad:
        w = I.Workload([ring])
        w.tasks = tasks
        assert oracle.run(I.single_batch(topo, w), 0)["rc"] == oracle.E_INVALID, tasks
