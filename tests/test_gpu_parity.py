"""Parity of the HIP megakernel (through the C ABI) with the CPU oracle.

All state is integer, so the bar is bit-exact equality: per experiment the
status, completion tick, packet-hops, delivered packets and flow digest; per
flow (recorded experiments) the arrival, activation and send-completion ticks.
"""

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from experiment_network_simulation_amd import inputs as I

pytestmark = pytest.mark.gpu

THREADS = min(16, os.cpu_count() or 1)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def simmod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from experiment_network_simulation_amd import sim
    sim.load_library()
    return sim


def oracle_all(oracle, batch, ids=None, flows=False):
    ob = oracle.OracleBatch(batch.pack())
    ids = list(range(batch.n_exp)) if ids is None else list(ids)
    with ThreadPoolExecutor(THREADS) as ex:
        return dict(zip(ids, ex.map(lambda e: oracle.run(ob, e, flows=flows), ids)))


def gpu_run(simmod, batch, record=(), force_global=False, max_ticks=0xFFFFFFF0, block_threads=0):
    s = simmod.Sim(batch, record=record, force_global=force_global, block_threads=block_threads)
    s.bind()
    s.run(max_ticks)
    return s, s.results()


def assert_exp(g, e, o, ge=None):
    ge = e if ge is None else ge
    assert o["rc"] == 0
    got = (int(g["status"][ge]), int(g["tick"][ge]), int(g["pkt_hops"][ge]), int(g["delivered"][ge]),
           int(g["digest"][ge]))
    want = (o["status"], o["t_end"], o["pkt_hops"], o["delivered"], o["digest"])
    assert got == want, f"experiment {e}: gpu {got} oracle {want}"


def assert_flows(s, ge, o):
    ft = s.flow_ticks(ge)
    for k in ("rd", "act", "sd"):
        bad = np.nonzero(ft[k] != o[k])[0]
        assert bad.size == 0, f"{k} differs at flows {bad[:8]} gpu {ft[k][bad[:8]]} oracle {o[k][bad[:8]]}"


# ------------------------------------------------------------ hand traces

@pytest.mark.parametrize("force_global", [False, True])
def test_hand_traces(simmod, oracle, force_global):
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_traces.json")))
    batch = I.Batch([], [], [], "hand")
    for name in ("M1_incast", "M2_credit", "M3_two_egress", "M4_round_order"):
        c = g[name]
        batch.topos.append(I.topology_from_cables(c["layers"], [tuple(x) for x in c["cables"]]))
        batch.works.append(I.xflows([tuple(f) for f in c["flows"]]))
        batch.exps.append(I.Experiment(len(batch.topos) - 1, len(batch.works) - 1, c["queue"], 0))
    s, r = gpu_run(simmod, batch, record=range(4), force_global=force_global)
    for e, name in enumerate(("M1_incast", "M2_credit", "M3_two_egress", "M4_round_order")):
        c = g[name]
        assert int(r["status"][e]) == 0 and int(r["tick"][e]) == c["t_end"]
        assert int(r["pkt_hops"][e]) == c["pkt_hops"]
        assert list(s.flow_ticks(e)["rd"]) == c["rd"]


# ------------------------------------------------------------ configs

@pytest.mark.parametrize("force_global", [False, True])
def test_c1_full(simmod, oracle, force_global):
    b = I.make_config(1)
    log("C1 full, force_global", force_global)
    s, r = gpu_run(simmod, b, record=range(16), force_global=force_global)
    o = oracle_all(oracle, b, flows=True)
    for e in range(16):
        assert_exp(r, e, o[e])
        assert_flows(s, e, o[e])


def test_c2_full(simmod, oracle):
    """All 256 experiments of the C2 batch in the default launch shape; per-flow
    ticks on a sample of experiments."""
    b = I.make_config(2)
    rec = [0, 7, 100, 255]
    log("C2 full batch")
    s, r = gpu_run(simmod, b, record=rec)
    o = oracle_all(oracle, b)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
    of = oracle_all(oracle, b, ids=rec, flows=True)
    for e in rec:
        assert_flows(s, e, of[e])


def test_c2_hbm_placement(simmod, oracle):
    b = I.make_config(2, n_exp=24)
    log("C2 first 24, HBM placement")
    s, r = gpu_run(simmod, b, record=[3], force_global=True)
    o = oracle_all(oracle, b)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
    assert_flows(s, 3, oracle.run(b, 3, flows=True))


def test_c3_full(simmod, oracle):
    b = I.make_config(3)
    rec = [0, 6, 27, 500, 1023]
    log("C3 full batch")
    s, r = gpu_run(simmod, b, record=rec)
    o = oracle_all(oracle, b)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
    of = oracle_all(oracle, b, ids=rec, flows=True)
    for e in rec:
        assert_flows(s, e, of[e])


@pytest.mark.parametrize("force_global", [False, True])
def test_c4_sample(simmod, oracle, force_global):
    """Two full-size k=8 fat-tree experiments (each ~93M packet-hops)."""
    ids = [2, 3]
    b = I.make_config(4, exp_ids=ids)
    log("C4 sample", ids, "force_global", force_global)
    s, r = gpu_run(simmod, b, record=[0], force_global=force_global)
    o = oracle_all(oracle, b, flows=False)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
    assert_flows(s, 0, oracle.run(b, 0, flows=True))


# C5 experiments spanning every oversubscription level (1, 2, 4) and the
# smallest and largest buffers the draw gives each (16/17 and 128 packets)
C5_IDS = [0, 1, 11, 134, 265, 294, 242, 43, 9, 2, 3, 4, 5, 6, 7, 8]


def test_c5_sample(simmod, oracle):
    """Sixteen full-size k=16 fat-tree experiments (6144 ports and 521,216 Zipf
    all-to-all flows each) on the general path, state in HBM: every
    oversubscription level, buffers of 16 to 128 packets."""
    b = I.make_config(5, exp_ids=C5_IDS)
    names = sorted({b.topos[x.topo].name for x in b.exps})
    assert names == ["fattree16o1", "fattree16o2", "fattree16o4"]
    qs = [x.queue_pkts for x in b.exps]
    assert min(qs) == 16 and max(qs) == 128
    log("C5 sample", [(b.topos[x.topo].name, x.queue_pkts) for x in b.exps])
    s, r = gpu_run(simmod, b, record=[0])
    o = oracle_all(oracle, b, flows=False)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
    assert_flows(s, 0, oracle.run(b, 0, flows=True))


@pytest.mark.parametrize("no_ring_path", [False, True])
def test_c4_stratified(simmod, oracle, no_ring_path):
    """C4 sampled evenly over the whole batch: every 64th of its 4096
    experiments (all NC, chunk and failure draws the batch holds), on the ring
    kernel and on the general compact kernel."""
    ids = list(range(0, 4096, 64))
    b = I.make_config(4, exp_ids=ids)
    log("C4 stratified", len(ids), "no_ring_path", no_ring_path)
    s = simmod.Sim(b, no_ring_path=no_ring_path)
    want = "msim_megakernel_c8h_r1" if no_ring_path else "msim_megakernel_ring"
    assert simmod.KERNEL_NAMES[s.info()["main_kernel"]] == want
    s.bind()
    s.run()
    r = s.results()
    o = oracle_all(oracle, b)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])


# ------------------------------------------------------------ semantics

def test_resume_equals_single_run(simmod, oracle):
    b = I.make_config(2, n_exp=8)
    s = simmod.Sim(b, record=[1])
    s.bind()
    rng = np.random.default_rng(0)
    steps = 0
    while True:
        s.run(int(rng.integers(1, 4000)))
        r = s.results()
        steps += 1
        if (r["status"] != 1).all():
            break
        # experiments still running report the ticks simulated so far
        assert steps < 200
    o = oracle_all(oracle, b)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
    assert_flows(s, 1, oracle.run(b, 1, flows=True))


@pytest.mark.parametrize("cid", [1, 2])
def test_general_path_resumed(simmod, oracle, cid):
    """The general path with its state in HBM, in random short runs: the
    per-tick pop counts (kept by tick parity), free-slot masks and queue
    slots carried across launch boundaries give the oracle's totals and
    flow ticks (C1: rate 1; C2: uplinks at rate 2)."""
    b = I.make_config(cid, n_exp=4)
    s = simmod.Sim(b, record=[1], force_global=True)
    s.bind()
    inf = s.info()
    assert inf["n_lds_exp"] == 0 and inf["lds_bytes"] == 0 and inf["main_kernel"] == 0
    rng = np.random.default_rng(cid)
    longest = {1: 100, 2: 3000}[cid]          # a few dozen runs per experiment
    for _ in range(400):
        s.run(int(rng.integers(1, longest)))
        r = s.results()
        if (r["status"] != 1).all():
            break
    o = oracle_all(oracle, b)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
    assert_flows(s, 1, oracle.run(b, 1, flows=True))


def test_incomplete_matches_oracle(simmod, oracle):
    b = I.make_config(1, n_exp=4)
    s, r = gpu_run(simmod, b, max_ticks=100)
    for e in range(4):
        o = oracle.run(b, e, max_ticks=100)
        assert int(r["status"][e]) == 1 and int(r["tick"][e]) == 100 == o["t_end"]
        assert int(r["pkt_hops"][e]) == o["pkt_hops"] and int(r["digest"][e]) == o["digest"]


def test_reset_and_rerun_is_deterministic(simmod):
    b = I.make_config(3, n_exp=28)
    s, r1 = gpu_run(simmod, b)
    s.reset()
    s.run()
    r2 = s.results()
    for k in ("status", "tick", "pkt_hops", "delivered", "digest"):
        assert np.array_equal(r1[k], r2[k])


def test_batch_composition_does_not_matter(simmod):
    """An experiment's result does not depend on what else is in the batch."""
    ids = [5, 9, 33, 120]
    solo = [gpu_run(simmod, I.make_config(2, exp_ids=[i]))[1] for i in ids]
    mixed = I.make_config(2, exp_ids=[120, 5, 33, 5, 9, 77])
    s, r = gpu_run(simmod, mixed)
    where = {120: 0, 5: 1, 33: 2, 9: 4}
    for i, so in zip(ids, solo):
        for k in ("status", "tick", "pkt_hops", "digest"):
            assert r[k][where[i]] == so[k][0]
    for k in ("tick", "digest"):
        assert r[k][1] == r[k][3]


def edge_batch():
    """Degenerate and extreme inputs mixed in one batch."""
    b = I.Batch([], [], [], "edges")

    def add(topo, work, q=16, seed=0):
        b.topos.append(topo)
        b.works.append(work)
        b.exps.append(I.Experiment(len(b.topos) - 1, len(b.works) - 1, q, seed))

    sw4 = I.single_switch(4)
    add(sw4, I.Workload())                                            # no traffic at all
    add(sw4, I.xflows([(0, 1, 1)]))                                   # one packet
    add(sw4, I.xflows([(0, 1, 5), (2, 1, 5), (3, 1, 5)]), q=1)        # incast with Q = 1
    fast = I.topology_from_cables([0, 0, 0, 1, 2], [(0, 3, 4, 4, 1, 1), (1, 3, 4, 4, 15, 1),
                                                    (3, 4, 4, 4, 7, 1), (2, 4, 3, 2, 2, 1)])
    add(fast, I.xflows([(0, 1, 40), (0, 2, 33), (1, 2, 17), (2, 0, 9)]), q=255)   # rate 4, delay 15
    add(fast, I.xflows([(0, 2, 50), (1, 2, 50)]), q=3)
    ls = I.leaf_spine(2, 4, 3, 1, 2, 3)
    add(ls, I.Workload([I.bcast(37 * I.PKT_BYTES, [7, 0, 4, 1, 5], 37)]), q=32)     # K = packets
    add(ls, I.Workload([I.ring(I.COLL_RING_AG, 203 * I.PKT_BYTES, [3, 6, 1], 3, 2 * I.PKT_BYTES),
                        I.ring(I.COLL_RING_AR, 77 * I.PKT_BYTES, [0, 5], 2, 5 * I.PKT_BYTES),
                        I.bcast(19 * I.PKT_BYTES, [2, 7, 4], 4)]), q=5, seed=12345)
    pairs = [(s, d, 1 + (3 * s + d) % 7) for s in range(8) for d in range(8) if s != d]
    add(ls, I.xflows(pairs), q=2, seed=99)                            # all-to-all, tiny buffers
    ft = I.fat_tree(4)
    ft.delay = np.asarray([1 + (c % 3) for c in range(ft.n_cables)], np.uint8)
    add(ft, I.Workload([I.ring(I.COLL_RING_AR, 64 * I.PKT_BYTES, [0, 5, 10, 15, 3, 8], 2, I.PKT_BYTES)]), q=4, seed=7)
    # deep buffers that fill: three senders at rate 4 (or 2) into one rate-1
    # output, so each ingress holds up to Q packets and slots past 64, 128 and
    # 192 (every word of a general-path free mask) are taken and returned
    deep4 = I.topology_from_cables([0, 0, 0, 0, 1], [(0, 4, 4, 4, 1, 1), (1, 4, 4, 4, 2, 1),
                                                     (2, 4, 4, 4, 1, 1), (3, 4, 1, 1, 1, 1)])
    add(deep4, I.xflows([(0, 3, 300), (1, 3, 280), (2, 3, 310)]), q=255)
    deep2 = I.topology_from_cables([0, 0, 0, 0, 1], [(0, 4, 2, 2, 1, 1), (1, 4, 2, 2, 1, 1),
                                                     (2, 4, 2, 2, 3, 1), (3, 4, 1, 1, 1, 1)])
    add(deep2, I.xflows([(0, 3, 200), (1, 3, 150), (2, 3, 170), (3, 0, 40)]), q=130)
    return b


@pytest.mark.parametrize("force_global", [False, True])
def test_edge_cases(simmod, oracle, force_global):
    b = edge_batch()
    s, r = gpu_run(simmod, b, record=range(b.n_exp), force_global=force_global)
    o = oracle_all(oracle, b, flows=True)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
        if o[e]["n_flows"]:
            assert_flows(s, e, o[e])
    assert int(r["tick"][0]) == 0 and int(r["status"][0]) == 0


def rate1_batch(n, seed):
    """Seeded experiments whose links all run at rate 1 (the compact kernels
    with per-tick pop counts, empty-queue head bytes and register free masks):
    per-cable delays 1..4, buffers of 1..64 packets (both sides of the 32-slot
    mask), 8- and 12-port switches, one to three rings with ragged channels, and
    every fourth experiment mixing in a broadcast and explicit flows."""
    rng = np.random.default_rng(seed)
    b = I.Batch([], [], [], "rate1")
    fabrics = [I.single_switch(8), I.single_switch(12), I.leaf_spine(3, 4, 2, 1, 1), I.fat_tree(4)]
    for f in fabrics:
        f.delay = rng.integers(1, 5, f.n_cables).astype(np.uint8)
        b.topos.append(f)
    queues = [1, 2, 5, 16, 31, 33, 64]
    for e in range(n):
        ti = e % len(fabrics)
        hosts = [int(x) for x in rng.permutation(b.topos[ti].hosts())]
        colls = []
        for _ in range(int(rng.integers(1, 4))):
            N = int(rng.integers(2, min(8, len(hosts)) + 1))
            members = [int(x) for x in rng.choice(hosts, N, replace=False)]
            nc = int(rng.integers(1, 4))
            P = nc * N * int(rng.integers(1, 5)) + int(rng.integers(0, N))
            kind = I.COLL_RING_AR if rng.integers(0, 2) else I.COLL_RING_AG
            colls.append(I.ring(kind, P * I.PKT_BYTES, members, nc, int(rng.integers(1, 6)) * I.PKT_BYTES))
        if e % 4 == 3:
            colls.append(I.bcast(23 * I.PKT_BYTES, hosts[:3], 4))
            w = I.xflows([(hosts[0], hosts[1], 7), (hosts[2], hosts[1], 5)])
            w.colls = colls
        else:
            w = I.Workload(colls)
        b.works.append(w)
        b.exps.append(I.Experiment(ti, len(b.works) - 1, queues[e % len(queues)], int(rng.integers(0, 2**32))))
    return b


def test_rate1_paths_one_run_and_resumed(simmod, oracle):
    """Rate-1 experiments run in one launch, and again resumed in random short
    runs (the pop counts, free masks and pending entries held in registers are
    saved and restored at every boundary): both match the oracle in every
    experiment's totals and every flow's ticks."""
    b = rate1_batch(24, 0x51)
    o = oracle_all(oracle, b, flows=True)
    s, r = gpu_run(simmod, b, record=range(b.n_exp))
    assert s.info()["n_compact"] == b.n_exp
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
        assert_flows(s, e, o[e])
    s2 = simmod.Sim(b, record=range(b.n_exp))
    s2.bind()
    rng = np.random.default_rng(7)
    for _ in range(400):
        s2.run(int(rng.integers(1, 40)))
        r2 = s2.results()
        if (r2["status"] != 1).all():
            break
    for e in range(b.n_exp):
        assert_exp(r2, e, o[e])
        assert_flows(s2, e, o[e])


@pytest.mark.parametrize("threads", [64, 256])
def test_block_size_does_not_matter(simmod, oracle, threads):
    """General path with fewer threads than ports (strided port loops)."""
    b = I.make_config(2, n_exp=6)
    s, r = gpu_run(simmod, b, block_threads=threads, force_global=True)
    o = oracle_all(oracle, b)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])


# -------------------------------------- tree, reduce-scatter, send/recv unit tasks

def collectives_batch(n, seed):
    """Small seeded mix of the further collective shapes on three fabrics, with
    random per-cable delays: trees of 2..16 members (1..3 channels, ragged last
    chunks), ring reduce-scatters, and unit tasks in all three send/recv
    strategies (the global all-gather gated on its scatter)."""
    rng = np.random.default_rng(seed)
    b = I.Batch([], [], [], "collectives")
    fabrics = [I.single_switch(12), I.leaf_spine(3, 4, 2), I.fat_tree(4)]
    for f in fabrics:
        f.delay = rng.integers(1, 4, f.n_cables).astype(np.uint8)
        b.topos.append(f)
    for e in range(n):
        ti = e % 3
        hosts = [int(x) for x in rng.permutation(b.topos[ti].hosts())]
        kind = (e // 3) % 3
        if kind == 0:
            N = int(rng.integers(2, min(12, len(hosts)) + 1))
            P, p = int(rng.integers(1, 90)), int(rng.integers(1, 12))
            colls = [I.tree(P * I.PKT_BYTES, hosts[:N], int(rng.integers(1, 4)) if P >= 3 else 1, p * I.PKT_BYTES)]
            if N + 3 <= len(hosts):
                colls.append(I.tree(40 * I.PKT_BYTES, hosts[N - 1:N + 3], 1, 3 * I.PKT_BYTES))
        elif kind == 1:
            N = int(rng.integers(2, 9))
            p = int(rng.integers(1, 5))
            colls = [I.ring(I.COLL_RING_RS, (N * p * int(rng.integers(1, 4)) + int(rng.integers(0, N))) * I.PKT_BYTES,
                            hosts[:N], int(rng.integers(1, 3)), p * I.PKT_BYTES)]
        else:
            A, B = int(rng.integers(1, 3)), int(rng.integers(1, 4))
            nodes = [hosts[1 + a * B:1 + (a + 1) * B] for a in range(A)]
            strat = ["sendrecv", "local_ag", "global_ag"][e % 3]
            P = A * B * int(rng.integers(1, 6))
            colls = I.unit_task(strat, P * I.PKT_BYTES, hosts[0], nodes, chunk_bytes=int(rng.integers(1, 3)) * I.PKT_BYTES)
        b.works.append(I.Workload(colls))
        b.exps.append(I.Experiment(ti, len(b.works) - 1, int(rng.integers(2, 20)), int(rng.integers(0, 2**32))))
    return b


@pytest.mark.parametrize("force_global", [False, True])
def test_collectives_mix(simmod, oracle, force_global):
    """Trees, reduce-scatters and unit tasks, every flow's ticks compared."""
    b = collectives_batch(27, 11)
    log("collectives mix", b.n_exp, "force_global", force_global)
    s, r = gpu_run(simmod, b, record=range(b.n_exp), force_global=force_global)
    o = oracle_all(oracle, b, flows=True)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
        assert_flows(s, e, o[e])


def test_collective_hand_traces_gpu(simmod, oracle):
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "collective_traces.json")))
    b = I.Batch([I.single_switch(3)], [], [], "collective traces")
    b.works.append(I.Workload([I.tree(2 * I.PKT_BYTES, [0, 1, 2], 1, 2 * I.PKT_BYTES)]))
    b.works.append(I.Workload(I.unit_task("global_ag", 4 * I.PKT_BYTES, 0, [[1], [2]], chunk_bytes=2 * I.PKT_BYTES)))
    b.exps = [I.Experiment(0, 0, 16, 0), I.Experiment(0, 1, 16, 0)]
    s, r = gpu_run(simmod, b, record=[0, 1])
    for e, name in enumerate(("T1_tree3", "T2_global_ag")):
        c = g[name]
        assert int(r["tick"][e]) == c["t_end"] and int(r["pkt_hops"][e]) == c["pkt_hops"]
        ft = s.flow_ticks(e)
        assert [int(x) for x in ft["rd"]] == c["rd"]
        assert [int(x) for x in ft["act"]] == c["act"]
        assert [int(x) for x in ft["sd"]] == c["sd"]


def test_c6_sample(simmod, oracle):
    """Full-size C6 experiments: a tree batch, two reduce-scatter batches and
    the three unit-task strategies."""
    ids = [0, 1, 2, 4, 5, 8]
    b = I.make_config(6, exp_ids=ids)
    log("C6 sample", ids)
    s, r = gpu_run(simmod, b, record=[2, 4, 5])
    o = oracle_all(oracle, b, flows=False)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
    for e in (2, 4, 5):
        assert_flows(s, e, oracle.run(b, e, flows=True))


# ------------------------------------------------------------ task graphs

def task_batch(n, seed):
    """Seeded task graphs: compute and intra-server tasks in chains and
    fork-joins, gating rings, trees, broadcasts and send/recv groups, beside
    collectives no task names, on three small fabrics."""
    rng = np.random.default_rng(seed)
    b = I.Batch([I.single_switch(8), I.leaf_spine(2, 4, 2), I.fat_tree(4)], [], [], "tasks")
    for e in range(n):
        ti = e % 3
        hosts = [int(x) for x in rng.permutation(b.topos[ti].hosts())]
        colls = []
        for j in range(int(rng.integers(1, 5))):
            kind = int(rng.integers(0, 4))
            mem = hosts[(3 * j) % 4: (3 * j) % 4 + int(rng.integers(2, 5))]
            if kind == 0:
                colls.append(I.ring(I.COLL_RING_AR, len(mem) * int(rng.integers(1, 9)) * I.PKT_BYTES, mem, 1, I.PKT_BYTES))
            elif kind == 1:
                colls.append(I.tree(int(rng.integers(1, 20)) * I.PKT_BYTES, mem, 1, 2 * I.PKT_BYTES))
            elif kind == 2:
                colls.append(I.bcast(int(rng.integers(2, 20)) * I.PKT_BYTES, mem, 2))
            else:
                colls.append(I.sendrecv(int(rng.integers(1, 6)) * I.PKT_BYTES, mem[0], mem[1:]))
        tasks = []
        for j in range(len(colls)):
            if rng.integers(0, 4) == 0:
                continue                              # this collective starts at tick 0
            preds = [int(q) for q in rng.choice(len(tasks), size=min(len(tasks), int(rng.integers(0, 3))),
                                                replace=False)] if tasks else []
            if rng.integers(0, 2):
                tasks.append(I.compute(int(rng.integers(1, 40)), preds))
            else:
                tasks.append(I.intra(int(rng.integers(0, 9)), int(rng.integers(1, 9000)), 1024, preds))
            tasks.append(I.comm(j, [len(tasks) - 1]))
        tasks.append(I.compute(int(rng.integers(1, 30)), list(range(len(tasks)))))
        w = I.Workload(colls)
        w.tasks = tasks
        b.works.append(w)
        b.exps.append(I.Experiment(ti, len(b.works) - 1, int(rng.integers(2, 16)), int(rng.integers(0, 2**32))))
    return b


@pytest.mark.parametrize("force_global", [False, True])
def test_task_graphs(simmod, oracle, force_global):
    """Every flow's and every task's ticks equal the oracle's."""
    b = task_batch(24, 21)
    log("task graphs", b.n_exp, "force_global", force_global)
    s, r = gpu_run(simmod, b, record=range(b.n_exp), force_global=force_global)
    o = oracle_all(oracle, b, flows=True)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
        assert_flows(s, e, o[e])
        tt = s.task_ticks(e)
        assert np.array_equal(tt["start"], o[e]["task_start"]) and np.array_equal(tt["finish"], o[e]["task_finish"])


def long_task_batch(n, seed):
    """task_batch with compute tasks of 100 to 2,000 ticks, so the network
    idles for long stretches between the phases of each graph."""
    b = task_batch(n, seed)
    rng = np.random.default_rng(seed + 1)
    for w in b.works:
        for tk in w.tasks:
            if tk.kind == I.TASK_COMPUTE:
                tk.ticks = int(rng.integers(100, 2000))
    return b


@pytest.mark.parametrize("force_global", [False, True])
def test_task_graphs_idle_network(simmod, oracle, force_global):
    """Where a task graph leaves the network empty the general path skips
    ticks: in one run, in random short runs, and in a run stopped inside an
    idle stretch, every flow's and every task's ticks (or the stopped state)
    equal the oracle's."""
    b = long_task_batch(12, 33)
    log("long task graphs", b.n_exp, "force_global", force_global)
    o = oracle_all(oracle, b, flows=True)
    s, r = gpu_run(simmod, b, record=range(b.n_exp), force_global=force_global)
    assert simmod.KERNEL_NAMES[s.info()["main_kernel"]] == "msim_megakernel_t"
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
        assert_flows(s, e, o[e])
        tt = s.task_ticks(e)
        assert np.array_equal(tt["start"], o[e]["task_start"]) and np.array_equal(tt["finish"], o[e]["task_finish"])
    s2 = simmod.Sim(b, record=range(b.n_exp), force_global=force_global)
    s2.bind()
    rng = np.random.default_rng(5)
    for _ in range(400):
        s2.run(int(rng.integers(1, 700)))
        r2 = s2.results()
        if (r2["status"] != 1).all():
            break
    for e in range(b.n_exp):
        assert_exp(r2, e, o[e])
        assert_flows(s2, e, o[e])
    stop = 1500
    s3, r3 = gpu_run(simmod, b, force_global=force_global, max_ticks=stop)
    for e in range(b.n_exp):
        oe = oracle.run(b, e, max_ticks=stop)
        got = (int(r3["status"][e]), int(r3["tick"][e]), int(r3["pkt_hops"][e]), int(r3["digest"][e]))
        assert got == (oe["status"], oe["t_end"], oe["pkt_hops"], oe["digest"]), f"experiment {e}"


def test_c7_sample(simmod, oracle):
    """Two full-size training iterations (tasks, intra-server collectives, DP
    all-reduce buckets on the k=8 fat-tree)."""
    b = I.make_config(7, exp_ids=[0, 1])
    log("C7 sample")
    s, r = gpu_run(simmod, b, record=[1])
    o = oracle_all(oracle, b, flows=True)
    for e in range(b.n_exp):
        assert_exp(r, e, o[e])
        tt = s.task_ticks(e)
        assert np.array_equal(tt["start"], o[e]["task_start"]) and np.array_equal(tt["finish"], o[e]["task_finish"])
    assert_flows(s, 1, o[1])


# ---------------------------------------------------------------------------
# Design-space exploration scored on the GPU (AutoCCL tuning, AlpaComm schedules)
# ---------------------------------------------------------------------------

def small_tune_tasks():
    """Five tuning tasks on C2's leaf-spine: 8 MiB all-reduces (ring and tree
    subspaces) over 16 hosts in seeded orders, and one all-gather."""
    topo = I.leaf_spine(4, 8, 4, host_rate=1, up_rate=2, delay=1)
    out = []
    for t in range(5):
        g = I.exp_rng(0x7E57, t)
        hosts = g.permutation(32)[:16]
        kind = I.COLL_RING_AG if t == 4 else I.COLL_RING_AR
        out.append(I.TuneTask(topo, kind, 8 * I.MIB, hosts, 32, g.u32()))
    return out


def test_autoccl_tuning_matches_oracle(simmod, oracle):
    from experiment_network_simulation_amd import dse as P
    from oracle import dse as D
    tasks = small_tune_tasks()
    starts = I.tune_starts(0x5A, len(tasks))
    ev = P.GpuEvaluator()
    got = P.tune(tasks, starts, ev)
    log(f"tuning: {ev.stats.batches} batches, {ev.stats.experiments} probes")
    with ThreadPoolExecutor(THREADS) as ex:
        refs = list(ex.map(lambda t: D.tune(tasks[t], starts[t]), range(len(tasks))))
    for t, ref in enumerate(refs):
        assert got[t].algo == ref["algo"] and got[t].ticks == ref["ticks"], t
        assert (got[t].nc, got[t].chunk) == (I.TUNE_NC[ref["best"][0]], I.TUNE_CHUNK[ref["best"][1]])
        for k, run in enumerate(ref["runs"]):
            assert got[t].per_subspace[k]["trace"] == run["probes"], (t, k)


def test_alpacomm_schedules_match_oracle(simmod, oracle):
    """Every scheduler's schedule on two resharding instances of a k=4
    fat-tree (mesh A hosts 0-7, mesh B hosts 8-15), scored on the GPU, against
    the oracle's schedulers and the oracle's simulation of each schedule."""
    from experiment_network_simulation_amd import dse as P
    from oracle import dse as D
    topo = I.fat_tree(4)
    K = 4
    insts = [(topo, I.resharding_tasks(s, n, range(8), range(8, 16), pkts_choices=(16, 32, 64)))
             for s, n in ((1, 6), (2, 10))]
    keys = [I.greedy_keys(100 + g, 10, 4) for g in range(3)]
    got = P.reshard(insts, K, keys, P.GpuEvaluator(), dfs_max_tasks=6)
    for (tp, tasks), r in zip(insts, got):
        ref = D.schedules(tasks, K, keys[0], with_dfs=len(tasks) <= 6)
        dur = P.durations(tasks, K)
        for name, s, t in zip(r.names, r.schedules, r.simulated):
            if name in ("naive", "load_balance", "greedy0"):
                rn = "greedy" if name == "greedy0" else name
                assert (s.sender, s.order) == (ref[rn]["sender"], ref[rn]["order"]), name
            if name.startswith("greedy") and name != "greedy0":
                g = D.greedy(tasks, dur, keys[int(name[6:])])
                assert (s.sender, s.order) == (g["sender"], g["order"]), name
            if name == "dfs":
                assert s.complete and s.makespan == ref["dfs"]["makespan"]
            o = D.simulate_schedule(tp, tasks, s.sender, s.order, K)
            assert int(t) == o["t_end"], (name, int(t), o["t_end"])
        log(f"reshard {len(tasks)} tasks: " + ", ".join(f"{n} {int(t)}" for n, t in zip(r.names, r.simulated)))


# ---------------------------------------------------------------------------
# Congestion control (ECN marks, ACK path, DCTCP windows)
# ---------------------------------------------------------------------------

def cc_batch(n, seed):
    """Rings, broadcasts, trees and explicit flows on three fabrics, DCTCP with
    thresholds and initial windows from tight to loose."""
    rng = np.random.default_rng(seed)
    topos = [I.single_switch(8), I.leaf_spine(2, 4, 2, host_rate=1, up_rate=2), I.fat_tree(4)]
    works, exps = [], []
    for e in range(n):
        t = e % 3
        nh = [8, 8, 16][t]
        hosts = [int(h) for h in rng.permutation(nh)]
        colls = [I.ring(I.COLL_RING_AR, 4 * 8 * I.PKT_BYTES * int(rng.integers(1, 4)), hosts[:4],
                        int(rng.integers(1, 3)), 2 * I.PKT_BYTES),
                 I.bcast(24 * I.PKT_BYTES, hosts[4:7], int(rng.choice([1, 4, 8])))]
        if t == 2:
            colls.append(I.tree(32 * I.PKT_BYTES, hosts[8:15], 2, 4 * I.PKT_BYTES))
        w = I.Workload(colls)
        pairs = [(hosts[i], hosts[(i + 3) % nh], int(rng.integers(1, 40))) for i in range(nh)]
        w.xsrc, w.xdst, w.xpkts = (np.array([p[k] for p in pairs], np.uint32) for k in range(3))
        works.append(w)
        K = int(rng.choice([0, 1, 2, 4, 8, 1000]))
        exps.append(I.Experiment(t, e, int(rng.integers(2, 17)), int(rng.integers(0, 2**32)), I.PKT_BYTES,
                                 I.CC_DCTCP, K, int(rng.choice([1, 2, 4, 16, 64]))))
    return I.Batch(topos, works, exps, "cc")


@pytest.mark.parametrize("force_global", [False, True])
def test_congestion_control(simmod, oracle, force_global):
    b = cc_batch(24, 13)
    s, g = gpu_run(simmod, b, record=range(b.n_exp), force_global=force_global)
    assert simmod.KERNEL_NAMES[s.info()["main_kernel"]] == "msim_megakernel_cc"
    ref = oracle_all(oracle, b, flows=True)
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
        assert_flows(s, e, ref[e])


def test_congestion_control_hand_traces_gpu(simmod, oracle):
    import json
    G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "cc_traces.json")))
    for name in ("AI_single_flow", "K0_window4", "incast_K1"):
        gd = G[name]
        b = I.single_batch(I.single_switch(gd["hosts"]), I.xflows([tuple(f) for f in gd["flows"]]), 16, 0,
                           cc=I.CC_DCTCP, ecn_k=gd["K"], cwnd0=gd["W0"])
        s, g = gpu_run(simmod, b, record=[0])
        ft = s.flow_ticks(0)
        assert list(ft["rd"]) == gd["rd"] and list(ft["sd"]) == gd["sd"], name
        assert int(g["tick"][0]) == max(gd["rd"])


def test_c8_sample(simmod, oracle):
    ids = [0, 101, 255]
    b = I.make_config(8, exp_ids=ids)
    s, g = gpu_run(simmod, b, record=[0])
    ref = oracle_all(oracle, b, flows=False)
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
    o = oracle.run(b, 0, flows=True)
    assert_flows(s, 0, o)


def dcqcn_batch(n, seed):
    """Rings, broadcasts, trees and explicit flows on three fabrics with DCQCN,
    thresholds from always-marking to never; every other experiment carries
    long explicit flows (timer and byte-counter stages), every fourth a long
    broadcast held back by a computation (timers due while idle)."""
    rng = np.random.default_rng(seed)
    topos = [I.single_switch(8), I.leaf_spine(2, 4, 2, host_rate=1, up_rate=2), I.fat_tree(4)]
    works, exps = [], []
    for e in range(n):
        t = e % 3
        nh = [8, 8, 16][t]
        hosts = [int(h) for h in rng.permutation(nh)]
        colls = [I.ring(I.COLL_RING_AR, 4 * 8 * I.PKT_BYTES * int(rng.integers(1, 4)), hosts[:4],
                        int(rng.integers(1, 3)), 2 * I.PKT_BYTES),
                 I.bcast(24 * I.PKT_BYTES, hosts[4:7], int(rng.choice([1, 4, 8])))]
        if t == 2:
            colls.append(I.tree(32 * I.PKT_BYTES, hosts[8:15], 2, 4 * I.PKT_BYTES))
        tasks = []
        if e % 4 == 1:
            colls.append(I.bcast(int(rng.integers(200, 1500)) * I.PKT_BYTES, [hosts[0], hosts[5]], 4))
            tasks = [I.compute(int(rng.integers(100, 1500))), I.comm(len(colls) - 1, [0])]
        w = I.Workload(colls)
        w.tasks = tasks
        top = 2500 if e % 2 == 0 else 40
        pairs = [(hosts[i], hosts[(i + 3) % nh], int(rng.integers(1, top))) for i in range(nh)]
        w.xsrc, w.xdst, w.xpkts = (np.array([p[k] for p in pairs], np.uint32) for k in range(3))
        works.append(w)
        K = int(rng.choice([0, 1, 2, 4, 8, 1000]))
        exps.append(I.Experiment(t, e, int(rng.integers(2, 17)), int(rng.integers(0, 2**32)), I.PKT_BYTES,
                                 I.CC_DCQCN, K, 0))
    return I.Batch(topos, works, exps, "dcqcn")


@pytest.mark.parametrize("force_global", [False, True])
def test_dcqcn(simmod, oracle, force_global):
    b = dcqcn_batch(24, 29)
    s, g = gpu_run(simmod, b, record=range(b.n_exp), force_global=force_global)
    assert simmod.KERNEL_NAMES[s.info()["main_kernel"]] == "msim_megakernel_cc"
    ref = oracle_all(oracle, b, flows=True)
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
        assert_flows(s, e, ref[e])


def test_dcqcn_pinned_scenarios_gpu(simmod, oracle):
    """The scenarios the oracle's DCQCN pins derive by hand (an always-marked
    flow, an incast with fast recovery, a second cut with additive and hyper
    increase, alpha decaying before a CNP), per flow on the GPU."""
    per = lambda P, src, dst: I.Workload([I.bcast(P * I.PKT_BYTES, [src, dst], P)])
    w1 = I.xflows([(0, 1, 538)])
    w2 = per(2000, 0, 2)
    w2.xsrc, w2.xdst, w2.xpkts = (np.array([v], np.uint32) for v in (1, 2, 2))
    w3 = per(40000, 0, 2)
    w3.xsrc, w3.xdst, w3.xpkts = (np.array([v], np.uint32) for v in (1, 2, 700))
    w4 = I.Workload([I.bcast(400 * I.PKT_BYTES, [0, 1], 400)])
    w4.tasks = [I.compute(5006), I.comm(0, [0])]
    topos = [I.single_switch(2), I.single_switch(3)]
    exps = [I.Experiment(0, 0, 16, 0, I.PKT_BYTES, I.CC_DCQCN, 0, 0),
            I.Experiment(1, 1, 16, 0, I.PKT_BYTES, I.CC_DCQCN, 1, 0),
            I.Experiment(1, 2, 16, 0, I.PKT_BYTES, I.CC_DCQCN, 1, 0),
            I.Experiment(0, 3, 16, 0, I.PKT_BYTES, I.CC_DCQCN, 0, 0)]
    b = I.Batch(topos, [w1, w2, w3, w4], exps, "dcqcn-pins")
    s, g = gpu_run(simmod, b, record=range(b.n_exp))
    ref = oracle_all(oracle, b, flows=True)
    assert [ref[0]["t_end"], ref[1]["t_end"]] == [1220 + 8 * 77 + 2, 2603]
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
        assert_flows(s, e, ref[e])


def test_c10_sample(simmod, oracle):
    ids = [0, 101, 255]
    b = I.make_config(10, exp_ids=ids)
    s, g = gpu_run(simmod, b, record=[0])
    ref = oracle_all(oracle, b, flows=False)
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
    o = oracle.run(b, 0, flows=True)
    assert_flows(s, 0, o)


def hpcc_batch(n, seed):
    """Rings, broadcasts, trees and explicit flows on three fabrics (links of
    rate 1 and 2, so telemetry of both rates) with HPCC; every other experiment
    carries long explicit flows, every fourth a broadcast held back by a
    computation."""
    rng = np.random.default_rng(seed)
    topos = [I.single_switch(8), I.leaf_spine(2, 4, 2, host_rate=1, up_rate=2), I.fat_tree(4)]
    works, exps = [], []
    for e in range(n):
        t = e % 3
        nh = [8, 8, 16][t]
        hosts = [int(h) for h in rng.permutation(nh)]
        colls = [I.ring(I.COLL_RING_AR, 4 * 8 * I.PKT_BYTES * int(rng.integers(1, 4)), hosts[:4],
                        int(rng.integers(1, 3)), 2 * I.PKT_BYTES),
                 I.bcast(24 * I.PKT_BYTES, hosts[4:7], int(rng.choice([1, 4, 8])))]
        if t == 2:
            colls.append(I.tree(32 * I.PKT_BYTES, hosts[8:15], 2, 4 * I.PKT_BYTES))
        tasks = []
        if e % 4 == 1:
            colls.append(I.bcast(int(rng.integers(200, 1500)) * I.PKT_BYTES, [hosts[0], hosts[5]], 4))
            tasks = [I.compute(int(rng.integers(100, 1500))), I.comm(len(colls) - 1, [0])]
        w = I.Workload(colls)
        w.tasks = tasks
        top = 2500 if e % 2 == 0 else 40
        pairs = [(hosts[i], hosts[(i + 3) % nh], int(rng.integers(1, top))) for i in range(nh)]
        w.xsrc, w.xdst, w.xpkts = (np.array([p[k] for p in pairs], np.uint32) for k in range(3))
        works.append(w)
        exps.append(I.Experiment(t, e, int(rng.integers(2, 17)), int(rng.integers(0, 2**32)), I.PKT_BYTES,
                                 I.CC_HPCC, 0, 0))
    return I.Batch(topos, works, exps, "hpcc")


@pytest.mark.parametrize("force_global", [False, True])
def test_hpcc(simmod, oracle, force_global):
    b = hpcc_batch(24, 31)
    s, g = gpu_run(simmod, b, record=range(b.n_exp), force_global=force_global)
    assert simmod.KERNEL_NAMES[s.info()["main_kernel"]] == "msim_megakernel_cc"
    ref = oracle_all(oracle, b, flows=True)
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
        assert_flows(s, e, ref[e])


def test_hpcc_pinned_scenarios_gpu(simmod, oracle):
    """The scenarios the oracle's HPCC pins derive by hand (a single flow's
    send ticks, an incast's first ticks), per flow on the GPU."""
    w1 = I.Workload([I.bcast(30 * I.PKT_BYTES, [0, 1], 30)])
    w2 = I.Workload([I.bcast(20 * I.PKT_BYTES, [0, 2], 20), I.bcast(20 * I.PKT_BYTES, [1, 2], 20)])
    exps = [I.Experiment(0, 0, 16, 0, I.PKT_BYTES, I.CC_HPCC, 0, 0),
            I.Experiment(1, 1, 16, 0, I.PKT_BYTES, I.CC_HPCC, 0, 0)]
    b = I.Batch([I.single_switch(2), I.single_switch(3)], [w1, w2], exps, "hpcc-pins")
    s, g = gpu_run(simmod, b, record=range(b.n_exp))
    ref = oracle_all(oracle, b, flows=True)
    assert list(np.asarray(ref[0]["sd"][:19], np.int64) - 1) == list(range(15)) + [16, 17, 18, 20]
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
        assert_flows(s, e, ref[e])


def test_c11_sample(simmod, oracle):
    ids = [0, 101, 255]
    b = I.make_config(11, exp_ids=ids)
    s, g = gpu_run(simmod, b, record=[0])
    ref = oracle_all(oracle, b, flows=False)
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
    o = oracle.run(b, 0, flows=True)
    assert_flows(s, 0, o)


# ---------------------------------------------------------------------------
# Packet spraying (per-packet equal-cost choice, in-order delivery)
# ---------------------------------------------------------------------------

def spray_batch(n, seed):
    """Rings, broadcasts, trees and explicit flows on multi-path fabrics (a
    k=4 fat-tree, an oversubscribed one, a two-spine leaf-spine with rate-2
    uplinks, random cable delays on some), every packet sprayed."""
    rng = np.random.default_rng(seed)
    topos = [I.fat_tree(4), I.fat_tree(4, oversub=2), I.leaf_spine(2, 4, 2, host_rate=1, up_rate=2)]
    slow = I.fat_tree(4)
    slow.delay = rng.integers(1, 5, slow.n_cables).astype(np.uint8)
    topos.append(slow)
    works, exps = [], []
    for e in range(n):
        t = e % 4
        nh = int((topos[t].layer == 0).sum())
        hosts = [int(h) for h in rng.permutation(nh)]
        colls = [I.ring(I.COLL_RING_AR, 4 * 8 * I.PKT_BYTES * int(rng.integers(1, 4)), hosts[:4],
                        int(rng.integers(1, 3)), 2 * I.PKT_BYTES),
                 I.bcast(32 * I.PKT_BYTES, hosts[4:7], int(rng.choice([1, 4, 8])))]
        if nh >= 16:
            colls.append(I.tree(32 * I.PKT_BYTES, hosts[8:15], 2, 4 * I.PKT_BYTES))
        w = I.Workload(colls)
        pairs = [(hosts[i], hosts[(i + 5) % nh], int(rng.integers(1, 60))) for i in range(nh)]
        w.xsrc, w.xdst, w.xpkts = (np.array([p[k] for p in pairs], np.uint32) for k in range(3))
        works.append(w)
        exps.append(I.Experiment(t, e, int(rng.integers(2, 17)), int(rng.integers(0, 2**32)), I.PKT_BYTES,
                                 lb=I.LB_SPRAY))
    return I.Batch(topos, works, exps, "spray")


@pytest.mark.parametrize("force_global", [False, True])
def test_packet_spraying(simmod, oracle, force_global):
    b = spray_batch(24, 31)
    s, g = gpu_run(simmod, b, record=range(b.n_exp), force_global=force_global)
    assert simmod.KERNEL_NAMES[s.info()["main_kernel"]] == "msim_megakernel_sp"
    ref = oracle_all(oracle, b, flows=True)
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
        assert_flows(s, e, ref[e])


def test_packet_spraying_closed_form_gpu(simmod, oracle):
    """The two-spine fabric of the oracle's pins: sprayed arrivals and
    in-order completions, on the GPU."""
    topo = I.topology_from_cables([0, 0, 1, 1, 2, 2], [(0, 2), (1, 3), (2, 4, 1, 1, 1), (2, 5, 1, 1, 5),
                                                       (3, 4, 1, 1, 1), (3, 5, 1, 1, 5)])
    f = oracle.fmix32
    for seed in (0, 1, 7, 123456789):
        P, K = 8, 4
        arrive = [j + (4 if 1 + f(f(j + 1) ^ f(2 ^ seed)) % 2 == 1 else 12) for j in range(P)]
        b = I.single_batch(topo, I.Workload([I.bcast(P * I.PKT_BYTES, [0, 1], K)]), 16, seed, lb=I.LB_SPRAY)
        s, g = gpu_run(simmod, b, record=[0])
        assert list(s.flow_ticks(0)["rd"]) == [max(arrive[:2 * (k + 1)]) for k in range(K)]


def test_c9_sample(simmod, oracle):
    ids = [0, 77, 200]
    b = I.make_config(9, exp_ids=ids)
    s, g = gpu_run(simmod, b, record=[0])
    ref = oracle_all(oracle, b, flows=False)
    for e in range(b.n_exp):
        assert_exp(g, e, ref[e])
    assert_flows(s, 0, oracle.run(b, 0, flows=True))
