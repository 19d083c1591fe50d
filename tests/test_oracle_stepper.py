"""The oracle against a brute-force stepper on an exhaustive grid of tiny cases.

tests/stepper.py writes the tick contract out literally (every port, every
flow and every queue visited every tick; all grants of a round decided before
any is applied) and shares no code with the oracle.  Where no closed form
reaches -- round-robin order and credit back-pressure under heavy mixing, ECMP
choices on multi-path fabrics, uneven channel and chunk splits -- the two must
agree on every flow's activation, last send and arrival tick.  The stepper
also runs with every phase visiting its entities in a random order: the
contract's pull discipline (Multiverse section 4.2: each egress pulls; one
writer per datum) makes the result independent of that order, which is what
lets the GPU run a phase's ports in parallel.
"""

import itertools
import json
import os
import random

import pytest

from experiment_network_simulation_amd import inputs as I

import stepper as S

PKT = I.PKT_BYTES
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_traces.json")


def same(oracle, b, e=0, shuffle=None):
    s = S.simulate(b, e, shuffle=shuffle)
    o = oracle.run(b, e, check=True, flows=True)
    assert o["rc"] == 0
    assert s["status"] == "done" and o["status"] == oracle.OK
    n = int(o["n_flows"])
    assert len(s["rd"]) == n
    assert [int(v) for v in o["rd"]] == s["rd"]
    assert [int(v) for v in o["act"]] == s["act"]
    assert [int(v) for v in o["sd"]] == s["sd"]
    assert o["t_end"] == s["t_end"]
    assert o["pkt_hops"] == s["pkt_hops"] and o["delivered"] == s["delivered"]
    assert o["max_occupancy"] == s["max_occupancy"]
    return s


def topology(kind, n_hosts, rate, delay):
    """Tiny fabrics: one switch; two switches on layers 1 and 2 joined by one
    cable (hosts alternate between them, so the cable is shared; a host cable
    may skip a layer); a leaf-spine with two spines (ECMP choices)."""
    if kind == "one":
        return I.single_switch(n_hosts, rate, delay)
    if kind == "two":
        layers = [0] * n_hosts + [1, 2]
        cables = [(h, n_hosts + (h % 2), 1, 1, delay, 1) for h in range(n_hosts)]
        cables.append((n_hosts, n_hosts + 1, rate, rate, delay, 1))
        return I.topology_from_cables(layers, cables)
    assert kind == "spine"
    per = (n_hosts + 1) // 2
    return I.leaf_spine(2, per, 2, 1, rate, delay)


def ring_bytes(N, NC, p):
    """A message whose channels differ by one packet and whose last rounds
    hold a remainder, so channel, round and chunk splits are all uneven."""
    return (NC * (N * p + N // 2 + 1) + NC - 1) * PKT


RING_GRID = list(itertools.product([2, 3, 4], [1, 2, 3], [1, 2, 3], [1, 2, 4], [1, 2], [1, 2],
                                   ["one", "two", "spine"], [I.COLL_RING_AR, I.COLL_RING_AG]))


def ring_case(N, NC, p, Q, d, r, topo_kind, kind):
    topo = topology(topo_kind, N if topo_kind != "spine" else 2 * ((N + 1) // 2), r, d)
    members = list(range(N))
    w = I.Workload([I.ring(kind, ring_bytes(N, NC, p), members, NC, p * PKT)])
    return I.single_batch(topo, w, queue_pkts=Q, ecmp_seed=N * 7 + NC * 3 + p)


@pytest.mark.parametrize("chunk", range(8))
def test_rings_exhaustive_grid(oracle, chunk):
    """N in {2,3,4}, NC in {1,2,3}, p in {1,2,3}, Q in {1,2,4}, delay in {1,2},
    rate in {1,2}, three fabrics, all-reduce and all-gather: 1,296 cases."""
    for case in RING_GRID[chunk::8]:
        same(oracle, ring_case(*case))


@pytest.mark.parametrize("A,K,P,Q,d,r,kind", list(itertools.product(
    [2, 3], [1, 2, 3], [5, 7], [1, 2, 4], [1, 2], [1, 2], ["one", "two", "spine"])))
def test_broadcast_grid(oracle, A, K, P, Q, d, r, kind):
    topo = topology(kind, 4, r, d)
    chain = [3, 0, 2, 1][:A + 1]
    b = I.single_batch(topo, I.Workload([I.bcast(P * PKT, chain, K)]), queue_pkts=Q, ecmp_seed=A + K)
    same(oracle, b)


@pytest.mark.parametrize("Q,d,r,kind", list(itertools.product([1, 2, 4], [1, 2], [1, 2], ["one", "two", "spine"])))
def test_incast_and_all_to_all(oracle, Q, d, r, kind):
    topo = topology(kind, 4, r, d)
    incast = I.xflows([(0, 3, 4), (1, 3, 2), (2, 3, 5)])
    b = I.single_batch(topo, incast, queue_pkts=Q, ecmp_seed=Q)
    same(oracle, b)
    a2a = I.xflows([(s, t, 1 + (s + 2 * t) % 3) for s in range(4) for t in range(4) if s != t])
    same(oracle, I.single_batch(topo, a2a, queue_pkts=Q, ecmp_seed=d))


@pytest.mark.parametrize("seed", range(24))
def test_mixed_workloads(oracle, seed):
    """Rings, broadcasts and explicit flows sharing hosts, NICs and links, so
    every host NIC round-robins over several connections."""
    rng = random.Random(seed)
    kind = ["one", "two", "spine"][seed % 3]
    topo = topology(kind, 4, rng.choice([1, 2]), rng.choice([1, 2]))
    colls = []
    for _ in range(rng.choice([1, 2])):
        N, NC, p = rng.choice([2, 3, 4]), rng.choice([1, 2, 3]), rng.choice([1, 2, 3])
        members = rng.sample(range(4), N)
        colls.append(I.ring(rng.choice([I.COLL_RING_AR, I.COLL_RING_AG, I.COLL_RING_RS]),
                            ring_bytes(N, NC, p), members, NC, p * PKT))
    chain = rng.sample(range(4), 3)
    colls.append(I.bcast(rng.choice([4, 5, 7]) * PKT, chain, rng.choice([1, 2, 3])))
    w = I.Workload(colls)
    pairs = [(s, t, rng.randint(1, 4)) for s in range(4) for t in range(4) if s != t and rng.random() < 0.4]
    x = I.xflows(pairs)
    w.xsrc, w.xdst, w.xpkts = x.xsrc, x.xdst, x.xpkts
    b = I.single_batch(topo, w, queue_pkts=rng.choice([1, 2, 4]), ecmp_seed=rng.getrandbits(32))
    same(oracle, b)


@pytest.mark.parametrize("seed", range(12))
def test_phase_order_does_not_matter(oracle, seed):
    """The same mixed cases with every phase of every tick visiting its ports,
    flows and grants in a random order: identical results, identical to the
    oracle."""
    rng = random.Random(100 + seed)
    case = RING_GRID[rng.randrange(len(RING_GRID))]
    b = ring_case(*case)
    base = S.simulate(b, 0)
    for k in range(3):
        got = S.simulate(b, 0, shuffle=random.Random(seed * 10 + k))
        assert got["rd"] == base["rd"] and got["act"] == base["act"] and got["sd"] == base["sd"]
    same(oracle, b, shuffle=random.Random(seed))


@pytest.mark.parametrize("case", ["M1_incast", "M2_credit", "M3_two_egress", "M4_round_order"])
def test_stepper_reproduces_hand_traces(case):
    """The stepper itself is pinned by the hand-derived traces."""
    g = json.load(open(GOLDEN))[case]
    topo = I.topology_from_cables(g["layers"], [tuple(c) for c in g["cables"]])
    b = I.single_batch(topo, I.xflows([tuple(f) for f in g["flows"]]), queue_pkts=g["queue"])
    s = S.simulate(b, 0)
    assert s["rd"] == g["rd"] and s["t_end"] == g["t_end"] and s["pkt_hops"] == g["pkt_hops"]


def test_stepper_ring_closed_form():
    """Contention-free ring, NC = 1, equal chunks: T = (R-1)((S-1)tau + p) + S tau
    with tau = L + p - 1 (the 2(N-1)-step count of AutoCCL section 4.1)."""
    for N, p, R, d, ag in [(3, 2, 3, 1, False), (4, 3, 2, 2, True), (5, 1, 2, 1, False)]:
        topo = I.single_switch(N, 1, d)
        kind = I.COLL_RING_AG if ag else I.COLL_RING_AR
        b = I.single_batch(topo, I.Workload([I.ring(kind, R * N * p * PKT, range(N), 1, p * PKT)]),
                           queue_pkts=d + 1)
        Ssteps = N - 1 if ag else 2 * (N - 1)
        tau = 2 * d + p - 1
        assert S.simulate(b, 0)["t_end"] == (R - 1) * ((Ssteps - 1) * tau + p) + Ssteps * tau


@pytest.mark.parametrize("seed", range(6))
def test_ecmp_routes_match(oracle, seed):
    """Every connection's path, port by port, from the stepper's own
    relaxation of up-then-down distances and its own hash
    (fmix32(key ^ fmix32(node ^ seed)), candidates in port order), against the
    oracle's, on a k=4 fat-tree, C4's k=8 fat-trees with failed cables, and a
    leaf-spine."""
    rng = random.Random(seed)
    if seed < 2:
        topo = I.fat_tree(4)
        hosts = list(range(16))
    elif seed < 4:
        b4 = I.make_config(4, exp_ids=[seed * 11 + 1])
        topo = b4.topos[b4.exps[0].topo]
        hosts = list(range(128))
    else:
        topo = I.leaf_spine(4, 4, 4, 1, 2, 1)
        hosts = list(range(16))
    pairs = [tuple(rng.sample(hosts, 2)) + (1,) for _ in range(40)]
    b = I.single_batch(topo, I.xflows(pairs), queue_pkts=8, ecmp_seed=rng.getrandbits(32))
    rc, pth = oracle.paths(b, 0)
    assert rc == 0
    ports = S._ports(topo)
    starts, k = [], 0
    for n in range(topo.n_nodes):
        starts.append(k)
        k += len(ports[n])
    for ci, (s, d, _) in enumerate(pairs):
        path = S._route(topo, ports, s, d, ci, b.exps[0].ecmp_seed)
        node, got = s, []
        for local in path:
            got.append(starts[node] + local)
            node = ports[node][local]["nbr"]
        want = [int(p) for p in pth["ports"][ci] if p != 0xFFFFFFFF]
        assert got == want, (ci, s, d)
