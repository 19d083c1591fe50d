"""Pins of the oracle's further collective shapes: the ring reduce-scatter, the
send/recv unit task and its strategies (with the gated all-gather), and the
binary-tree all-reduce.

Every expected value is computed independently of the oracle's code: hand
traces (tests/golden/collective_traces.json), closed forms derived from the
tick rules, and the predecessor rules rebuilt here from their definitions,
checked through activation ticks (a flow activates exactly at the first tick
by which all of its predecessors are met: RD for RECV, SD for SEND).
"""

import json
import os

import numpy as np
import pytest

from experiment_network_simulation_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "collective_traces.json")
PKT = I.PKT_BYTES


def ceil_div(a, b):
    return -(-a // b)


def check_activation(r, preds):
    """preds[f] = list of (flow, 'R' | 'S'); activation = latest predecessor tick."""
    for f, ps in enumerate(preds):
        want = max((int(r["rd"][g]) if k == "R" else int(r["sd"][g]) for g, k in ps), default=0)
        assert int(r["act"][f]) == want, (f, ps)


# ------------------------------------------------------------ hand traces

def _trace_workload(case):
    if case == "T1_tree3":
        return I.Workload([I.tree(2 * PKT, [0, 1, 2], 1, 2 * PKT)])
    return I.Workload(I.unit_task("global_ag", 4 * PKT, 0, [[1], [2]], chunk_bytes=2 * PKT))


@pytest.mark.parametrize("case", ["T1_tree3", "T2_global_ag"])
def test_collective_hand_traces(oracle, case):
    g = json.load(open(GOLDEN))[case]
    b = I.single_batch(I.single_switch(g["hosts"]), _trace_workload(case), queue_pkts=16)
    r = oracle.run(b, 0, check=True, flows=True)
    assert r["status"] == oracle.OK
    assert [int(x) for x in r["rd"]] == g["rd"]
    assert [int(x) for x in r["act"]] == g["act"]
    assert [int(x) for x in r["sd"]] == g["sd"]
    assert r["t_end"] == g["t_end"] and r["pkt_hops"] == g["pkt_hops"]


# ------------------------------------------------------------------ tree

def tree_pair_closed_form(P, p, L):
    """Two members, R = ceil(P/p) chunks, the last of X = P - (R-1)p packets.
    Up chunk k leaves the child during [kp, kp + size_k) and lands L - 1 ticks
    after its last packet; down chunk k starts when up chunk k has landed and
    down chunk k-1 has left, which for full chunks is (k+1)p - 1 + L (both
    bounds meet); the last down chunk starts at Rp - 1 + L (R > 1) or
    X - 1 + L (R = 1) and lands X - 1 + L ticks later."""
    R = ceil_div(P, p)
    X = P - (R - 1) * p
    start = X - 1 + L if R == 1 else R * p - 1 + L
    return start + X - 1 + L


@pytest.mark.parametrize("P,p,d", [(1, 1, 1), (5, 2, 1), (8, 4, 2), (7, 3, 3), (12, 12, 1), (40, 6, 2)])
def test_tree_pair_closed_form(oracle, P, p, d):
    """Up and down use opposite directions of the same cables, so nothing contends."""
    w = I.Workload([I.tree(P * PKT, [1, 0], 1, p * PKT)])
    b = I.single_batch(I.single_switch(2, 1, d), w, queue_pkts=d + 1)
    r = oracle.run(b, 0, check=True)
    assert r["status"] == oracle.OK
    assert r["t_end"] == tree_pair_closed_form(P, p, 2 * d)
    R = ceil_div(P, p)
    assert r["n_flows"] == 2 * R and r["delivered"] == 2 * P


def tree_preds(N, NC, P, p):
    """Rule W7, rebuilt: per channel, connections up(i) = i-1 and down(i) =
    N-1+i-1 for nodes i = 1..N-1; flow (chunk k, connection j) = base + k E + j
    with E = 2(N-1).  Returns (preds, sizes)."""
    preds, sizes = [], []
    E = 2 * (N - 1)
    children = lambda i: [c for c in (2 * i + 1, 2 * i + 2) if c < N]
    for c in range(NC):
        Pc = P // NC + (1 if c < P % NC else 0)
        R = ceil_div(Pc, p)
        base = len(preds)
        for k in range(R):
            for j in range(E):
                ps = []
                fk = base + k * E
                if j < N - 1:
                    i = j + 1
                    ps += [(fk + ch - 1, "R") for ch in children(i)]
                else:
                    i = j - (N - 1) + 1
                    par = (i - 1) // 2
                    if par == 0:
                        ps += [(fk + ch - 1, "R") for ch in children(0)]
                    else:
                        ps.append((fk + (N - 1) + par - 1, "R"))
                if k >= 1:
                    ps.append((fk - E + j, "S"))
                preds.append(ps)
                sizes.append(p if k + 1 < R else Pc - (R - 1) * p)
    return preds, sizes


@pytest.mark.parametrize("N,NC,P,p,topo", [(3, 1, 6, 2, "switch"), (5, 2, 23, 3, "switch"),
                                           (7, 1, 16, 4, "leafspine"), (8, 3, 40, 5, "fattree"),
                                           (2, 1, 9, 9, "switch"), (16, 2, 64, 8, "fattree")])
def test_tree_dependencies_and_sizes(oracle, N, NC, P, p, topo):
    """Every flow of the tree activates exactly when its W7 predecessors are met,
    flow sizes follow the chunk split, and the usual bounds hold."""
    t = {"switch": I.single_switch(N), "leafspine": I.leaf_spine(2, 4, 2),
         "fattree": I.fat_tree(4)}[topo]
    rng = np.random.default_rng(N * 100 + P)
    members = [int(x) for x in rng.permutation(t.hosts())[:N]]
    w = I.Workload([I.tree(P * PKT, members, NC, p * PKT)])
    b = I.single_batch(t, w, queue_pkts=8, ecmp_seed=7)
    r = oracle.run(b, 0, check=True, flows=True)
    assert r["status"] == oracle.OK
    preds, sizes = tree_preds(N, NC, P, p)
    rc, fl = oracle.flows(b, 0)
    assert rc == 0 and [int(s) for s in fl["size"]] == sizes
    check_activation(r, preds)
    # every member receives the whole message once (down), every non-root sends it up once
    assert r["delivered"] == 2 * (N - 1) * P


# ------------------------------------------------------- send/recv unit task

@pytest.mark.parametrize("A,P,d", [(1, 3, 1), (3, 4, 1), (4, 2, 2), (6, 1, 3), (5, 17, 1)])
def test_sendrecv_closed_form(oracle, A, P, d):
    """Sequential sends (W6): flow j starts when flow j-1 has left (jP), sends
    P packets and lands 2d - 1 ticks after its last send: RD_j = (j+1)P + 2d - 1,
    the tick form of T_sr = A t for A receivers."""
    w = I.Workload([I.sendrecv(P * PKT, 0, range(1, A + 1))])
    b = I.single_batch(I.single_switch(A + 1, 1, d), w, queue_pkts=d + 1)
    r = oracle.run(b, 0, check=True, flows=True)
    assert r["status"] == oracle.OK
    for j in range(A):
        assert int(r["act"][j]) == j * P
        assert int(r["sd"][j]) == (j + 1) * P
        assert int(r["rd"][j]) == (j + 1) * P + 2 * d - 1
    assert r["t_end"] == A * P + 2 * d - 1


@pytest.mark.parametrize("A,B,P", [(2, 2, 8), (3, 2, 12), (4, 1, 5), (2, 4, 16)])
def test_unit_task_strategy_closed_forms(oracle, A, B, P):
    """AlpaComm's send/recv and local all-gather strategies in ticks, for a
    slice of P packets: the source link carries A B slices (T_sr = A B t) or
    A B parts of P / B packets, i.e. A slices (T_srla = A t), plus the last
    packet's path latency L - 1 (one switch, delay 1: L = 2)."""
    nodes = [[1 + a * B + i for i in range(B)] for a in range(A)]
    topo = I.single_switch(1 + A * B)
    for strategy, T in (("sendrecv", A * B * P + 1), ("local_ag", A * P + 1)):
        w = I.Workload(I.unit_task(strategy, P * PKT, 0, nodes))
        r = oracle.run(I.single_batch(topo, w, queue_pkts=4), 0, check=True)
        assert r["status"] == oracle.OK and r["t_end"] == T, strategy


@pytest.mark.parametrize("A,B,P,p", [(2, 2, 8, 1), (2, 3, 12, 2), (3, 2, 24, 2)])
def test_global_ag_dependencies(oracle, A, B, P, p):
    """The global all-gather strategy: parts of P/(A B) packets go out in turn,
    then a ring all-gather of the slice in which rank i's first step waits on
    the arrival of part i (and on nothing else), the rest following W1."""
    nodes = [[1 + a * B + i for i in range(B)] for a in range(A)]
    N = A * B
    topo = I.leaf_spine(2, 4, 2) if N + 1 > 4 else I.single_switch(N + 1)
    hosts = list(range(N + 1))
    w = I.Workload(I.unit_task("global_ag", P * PKT, hosts[0], nodes, chunk_bytes=p * PKT))
    b = I.single_batch(topo, w, queue_pkts=8, ecmp_seed=3)
    r = oracle.run(b, 0, check=True, flows=True)
    assert r["status"] == oracle.OK
    preds = [[] if j == 0 else [(j - 1, "S")] for j in range(N)]
    S = N - 1
    R = ceil_div(P, N * p)
    if R > 1 and P - (R - 1) * N * p < N:
        R -= 1
    fid = lambda rr, s, i: N + (rr * S + s) * N + i
    for rr in range(R):
        for s in range(S):
            for i in range(N):
                if s >= 1:
                    preds.append([(fid(rr, s - 1, (i - 1) % N), "R"), (fid(rr, s - 1, i), "S")])
                elif rr >= 1:
                    preds.append([(fid(rr - 1, S - 1, i), "S")])
                else:
                    preds.append([(i, "R")])
    assert len(preds) == len(r["act"])
    check_activation(r, preds)


def test_gate_validation(oracle):
    """A gate must name an earlier send/recv whose receivers are the ring's members, in order."""
    topo = I.single_switch(4)
    part = I.sendrecv(2 * PKT, 0, [1, 2, 3])
    ok = I.ring(I.COLL_RING_AG, 6 * PKT, [1, 2, 3], 1, PKT)
    ok.gate = 0
    assert oracle.run(I.single_batch(topo, I.Workload([part, ok])), 0)["rc"] == 0
    for bad_members, gate in (([2, 1, 3], 0), ([1, 2], 0), ([1, 2, 3], 1)):
        g = I.ring(I.COLL_RING_AG, 6 * PKT, bad_members, 1, PKT)
        g.gate = gate
        r = oracle.run(I.single_batch(topo, I.Workload([part, g])), 0)
        assert r["rc"] == oracle.E_INVALID, (bad_members, gate)
    twice = I.ring(I.COLL_RING_RS, 6 * PKT, [1, 2, 3], 1, PKT)
    twice.gate = 0
    assert oracle.run(I.single_batch(topo, I.Workload([part, ok, twice])), 0)["rc"] == oracle.E_INVALID


# ------------------------------------------------------ ring reduce-scatter

@pytest.mark.parametrize("N,p,R,NC", [(4, 2, 1, 1), (4, 3, 2, 1), (6, 1, 3, 1), (5, 2, 2, 3)])
def test_reduce_scatter_is_allgather_shaped(oracle, N, p, R, NC):
    """With a reduction that costs no time, the ring reduce-scatter moves the
    same chunks along the same ring as the all-gather of the same size
    (N - 1 steps, chunk (i - s) mod N): identical per-flow ticks, and the NC = 1
    closed form (R-1)((N-2)tau + p) + (N-1)tau with tau = L + p - 1."""
    topo = I.single_switch(N)
    P = R * N * p * NC
    out = []
    for kind in (I.COLL_RING_RS, I.COLL_RING_AG):
        w = I.Workload([I.ring(kind, P * PKT, range(N), NC, p * PKT)])
        r = oracle.run(I.single_batch(topo, w, queue_pkts=2), 0, check=True, flows=True)
        assert r["status"] == oracle.OK
        out.append(r)
    for k in ("rd", "act", "sd"):
        assert np.array_equal(out[0][k], out[1][k])
    if NC == 1:
        tau = 2 + p - 1
        assert out[0]["t_end"] == (R - 1) * ((N - 2) * tau + p) + (N - 1) * tau
