"""The C-ABI library loads, exports every entry point include/msim.h declares,
and its host-side compile (validation, routing, flow expansion) behaves, all
without a GPU."""

import os
import re
import subprocess

import numpy as np
import pytest

from experiment_network_simulation_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msim.h")


@pytest.fixture(scope="module")
def simmod():
    from experiment_network_simulation_amd import sim
    sim.load_library()
    return sim


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char \*)\s*(msim_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(simmod):
    names = declared_functions()
    assert len(names) >= 11
    out = subprocess.run(["nm", "-D", "--defined-only", simmod.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in names:
        assert n in exported, n
    assert sorted(names) == sorted(simmod.EXPORTED)


def test_create_reports_sizes(simmod):
    s = simmod.Sim(I.make_config(1))
    inf = s.info()
    # compact path: 8 host slots padded to a 64-wide wavefront, then 8 switch ports
    assert inf["n_exp"] == 16 and inf["n_compact"] == 16 and inf["block_threads"] == 128
    assert inf["max_ports"] == 16
    assert inf["est_pkt_hops"] == 16 * 7168 and inf["est_delivered"] == 16 * 3584
    assert s.workspace_bytes > 0
    assert [s.flow_count(e) for e in range(4)] == [896, 448, 224, 112]


def test_general_layouts_keep_their_sides(simmod):
    # The general kernels address the switch and NIC state as LDS and the
    # per-connection state as global memory when only the former fits in LDS,
    # taking each array's side from the layout order; msim_create checks every
    # array's side and fails otherwise.  Every general-path kind compiles here:
    # plain (C5, k=16 fat-tree), task graph (C7), DCTCP (C8), spraying (C9),
    # DCQCN (C10), HPCC (C11).
    for cid, kind in [(5, 0), (7, 9), (8, 10), (9, 13), (10, 10), (11, 10)]:
        s = simmod.Sim(I.make_config(cid, n_exp=2))
        inf = s.info()
        assert inf["n_exp"] == 2 and inf["n_compact"] == 0 and inf["main_kernel"] == kind, (cid, inf)


def test_ring_staging_slots_for_every_c4_experiment(simmod):
    # The ring layout permutes the staging words so that every wavefront's
    # reads and writes fall in 64 different LDS banks; msim_create builds the
    # edge colouring and checks it (one word per port, below the padded slot
    # count, 64 banks per wavefront on both sides), failing otherwise.  All
    # 4096 C4 experiments (failed cables included) and C1 take the ring path.
    for cid, n in [(1, 16), (4, 4096)]:
        s = simmod.Sim(I.make_config(cid))
        inf = s.info()
        assert inf["n_exp"] == n and simmod.KERNEL_NAMES[inf["main_kernel"]] == "msim_megakernel_ring", (cid, inf)


def test_flow_counts_match_oracle(simmod, oracle):
    for cid, n in [(2, 6), (3, 28)]:
        b = I.make_config(cid, n_exp=n)
        s = simmod.Sim(b)
        for e in range(n):
            rc, nf, nc = oracle.count(b, e)
            assert rc == 0 and s.flow_count(e) == nf


def test_packet_hop_estimate_matches_oracle_paths(simmod, oracle):
    """The host compile's sum of flow size x path links equals the oracle's."""
    b = I.make_config(4, exp_ids=[0, 1, 2])
    s = simmod.Sim(b)
    tot = 0
    for e in range(3):
        rc, fl = oracle.flows(b, e)
        rc2, pth = oracle.paths(b, e)
        tot += int((fl["size"].astype(np.int64) * pth["links"][fl["conn"]]).sum())
    assert s.info()["est_pkt_hops"] == tot


def expect_error(simmod, batch, code):
    with pytest.raises(simmod.MsimError) as ei:
        simmod.Sim(batch)
    assert ei.value.code == code


def test_validation_errors(simmod):
    topo = I.single_switch(3)
    # dead host cable -> unroutable
    t2 = topo.copy(); t2.alive[1] = 0
    expect_error(simmod, I.single_batch(t2, I.xflows([(0, 1, 2)])), simmod.E_UNROUTABLE)
    # too few packets per channel
    w = I.Workload([I.ring(I.COLL_RING_AR, 2 * I.PKT_BYTES, range(3), 1, I.PKT_BYTES)])
    expect_error(simmod, I.single_batch(topo, w), simmod.E_INVALID_SPEC)
    # chunk not a whole number of packets
    w = I.Workload([I.ring(I.COLL_RING_AR, 64 * I.PKT_BYTES, range(3), 1, 100)])
    expect_error(simmod, I.single_batch(topo, w), simmod.E_INVALID_SPEC)
    # queue out of range
    expect_error(simmod, I.single_batch(topo, I.xflows([(0, 1, 2)]), queue_pkts=0), simmod.E_INVALID_SPEC)
    expect_error(simmod, I.single_batch(topo, I.xflows([(0, 1, 2)]), queue_pkts=256), simmod.E_INVALID_SPEC)
    # same-layer cable
    bad = I.topology_from_cables([0, 1, 1], [(0, 1), (1, 2)])
    expect_error(simmod, I.single_batch(bad, I.Workload()), simmod.E_INVALID_SPEC)
    # host with two cables
    bad = I.topology_from_cables([0, 1, 2], [(0, 1), (0, 2), (1, 2)])
    expect_error(simmod, I.single_batch(bad, I.Workload()), simmod.E_INVALID_SPEC)
    # rate and delay limits
    bad = I.topology_from_cables([0, 0, 1], [(0, 2, 5, 1, 1, 1), (1, 2)])
    expect_error(simmod, I.single_batch(bad, I.Workload()), simmod.E_INVALID_SPEC)
    bad = I.topology_from_cables([0, 0, 1], [(0, 2, 1, 1, 16, 1), (1, 2)])
    expect_error(simmod, I.single_batch(bad, I.Workload()), simmod.E_INVALID_SPEC)
    # repeated ring member, broadcast K > packets, explicit flow to itself
    w = I.Workload([I.ring(I.COLL_RING_AR, 64 * I.PKT_BYTES, [0, 1, 1], 1, I.PKT_BYTES)])
    expect_error(simmod, I.single_batch(topo, w), simmod.E_INVALID_SPEC)
    w = I.Workload([I.bcast(4 * I.PKT_BYTES, [0, 1], 5)])
    expect_error(simmod, I.single_batch(topo, w), simmod.E_INVALID_SPEC)
    expect_error(simmod, I.single_batch(topo, I.xflows([(1, 1, 2)])), simmod.E_INVALID_SPEC)
    # switch with more than 16 ports
    big = I.single_switch(17)
    expect_error(simmod, I.single_batch(big, I.Workload()), simmod.E_LIMIT)


def test_bind_without_workspace_is_rejected(simmod):
    s = simmod.Sim(I.make_config(1, n_exp=1))
    lib = simmod.load_library()
    import ctypes as C
    rc = lib.msim_bind(s._ctx, None, 0, None)
    assert rc == simmod.E_WORKSPACE
    assert lib.msim_run(s._ctx, 10, None, 0) == simmod.E_STATE
    assert b"before msim_bind" in lib.msim_last_error(s._ctx)


def test_workspace_covers_flow_records(simmod):
    """Recording per-flow ticks (rd, act, sd: 3 x 4 bytes per flow) grows the
    workspace by at least that much (regression: the record area once fell
    outside the reported size)."""
    b = I.make_config(2, n_exp=8)
    plain = simmod.Sim(b).workspace_bytes
    rec = [0, 3, 7]
    s = simmod.Sim(b, record=rec)
    assert s.workspace_bytes >= plain + 12 * sum(s.flow_count(e) for e in rec)


def test_further_collectives_compile(simmod, oracle):
    """Trees, reduce-scatters and send/recv unit tasks: flow counts equal the
    oracle's; all of them run compact, the trees and unit tasks on the kernel
    that carries those rules, and with force_global none does."""
    b = I.make_config(6, exp_ids=list(range(9)))
    s = simmod.Sim(b)
    for e in range(b.n_exp):
        rc, nf, nc = oracle.count(b, e)
        assert rc == 0 and s.flow_count(e) == nf
    inf = s.info()
    assert inf["n_compact"] == 9
    assert simmod.KERNEL_NAMES[inf["main_kernel"]] == "msim_megakernel_c8h_r1_x"   # 6 of the 9
    rs = simmod.Sim(b.subset([1, 4, 7]))                                           # reduce-scatters only
    assert simmod.KERNEL_NAMES[rs.info()["main_kernel"]] == "msim_megakernel_ring"
    assert simmod.Sim(b, force_global=True).info()["n_compact"] == 0


def test_gate_validation_errors(simmod):
    topo = I.single_switch(5)
    part = I.sendrecv(2 * I.PKT_BYTES, 0, [1, 2, 3])
    for members, gate, first in (([2, 1, 3], 0, part), ([1, 2], 0, part), ([1, 2, 3], 1, part),
                                 ([1, 2, 3], 0, I.bcast(2 * I.PKT_BYTES, [0, 1, 2, 3], 1))):
        ag = I.ring(I.COLL_RING_AG, 6 * I.PKT_BYTES, members, 1, I.PKT_BYTES)
        ag.gate = gate
        expect_error(simmod, I.single_batch(topo, I.Workload([first, ag])), simmod.E_INVALID_SPEC)
    # a send/recv gates one collective only
    a1 = I.ring(I.COLL_RING_AG, 6 * I.PKT_BYTES, [1, 2, 3], 1, I.PKT_BYTES)
    a2 = I.ring(I.COLL_RING_RS, 6 * I.PKT_BYTES, [1, 2, 3], 1, I.PKT_BYTES)
    a1.gate = a2.gate = 0
    expect_error(simmod, I.single_batch(topo, I.Workload([part, a1, a2])), simmod.E_INVALID_SPEC)
    # trees need whole-packet chunks, send/recv at least one packet
    w = I.Workload([I.tree(8 * I.PKT_BYTES, [0, 1, 2], 1, 100)])
    expect_error(simmod, I.single_batch(topo, w), simmod.E_INVALID_SPEC)
    w = I.Workload([I.sendrecv(0, 0, [1, 2])])
    expect_error(simmod, I.single_batch(topo, w), simmod.E_INVALID_SPEC)


def test_task_graph_compile_and_validation(simmod, oracle):
    """Task graphs compile onto the general task kernel, and invalid graphs are
    rejected as the oracle rejects them."""
    b = I.make_config(7, exp_ids=[0, 3])
    s = simmod.Sim(b)
    inf = s.info()
    assert inf["n_compact"] == 0 and simmod.KERNEL_NAMES[inf["main_kernel"]] == "msim_megakernel_t"
    for e in range(b.n_exp):
        assert s.task_count(e) == len(b.works[b.exps[e].work].tasks)
        assert s.flow_count(e) == oracle.count(b, e)[1]
    topo = I.single_switch(4)
    ring = I.ring(I.COLL_RING_AG, 4 * I.PKT_BYTES, range(4), 1, I.PKT_BYTES)
    for tasks in ([I.compute(0)], [I.compute(2, [0])], [I.comm(1)], [I.comm(0), I.comm(0)],
                  [I.intra(0, 0, 5)], [I.intra(1, 10, 0)]):
        w = I.Workload([ring])
        w.tasks = tasks
        expect_error(simmod, I.single_batch(topo, w), simmod.E_INVALID_SPEC)
        assert oracle.run(I.single_batch(topo, w), 0)["rc"] == oracle.E_INVALID


def test_congestion_control_compile_and_validation(simmod, oracle):
    """Experiments with DCTCP compile onto the congestion-control kernel (the
    same batch without it stays compact), and bad parameters are rejected as
    the oracle rejects them."""
    b = I.make_config(8, exp_ids=[0, 5])
    s = simmod.Sim(b)
    inf = s.info()
    assert inf["n_compact"] == 0 and simmod.KERNEL_NAMES[inf["main_kernel"]] == "msim_megakernel_cc"
    for e in range(b.n_exp):
        assert s.flow_count(e) == oracle.count(b, e)[1]
    for x in b.exps:
        x.cc = I.CC_NONE
    assert simmod.Sim(b).info()["n_compact"] == 2
    topo = I.single_switch(2)
    w = I.xflows([(0, 1, 3)])
    for cc, k, w0 in ((I.CC_DCTCP, 1, 0), (I.CC_DCTCP, 1, 65536), (4, 1, 1)):
        bb = I.single_batch(topo, w, cc=cc, ecn_k=k, cwnd0=w0)
        expect_error(simmod, bb, simmod.E_INVALID_SPEC)
        assert oracle.run(bb, 0)["rc"] == oracle.E_INVALID


def test_dcqcn_compile_and_validation(simmod, oracle):
    """DCQCN experiments compile onto the congestion-control kernel; DCQCN with
    spraying is rejected as the oracle rejects it."""
    b = I.make_config(10, exp_ids=[0, 7])
    s = simmod.Sim(b)
    inf = s.info()
    assert inf["n_compact"] == 0 and simmod.KERNEL_NAMES[inf["main_kernel"]] == "msim_megakernel_cc"
    for e in range(b.n_exp):
        assert s.flow_count(e) == oracle.count(b, e)[1]
    bb = I.single_batch(I.single_switch(2), I.xflows([(0, 1, 3)]), cc=I.CC_DCQCN, ecn_k=2, lb=I.LB_SPRAY)
    expect_error(simmod, bb, simmod.E_INVALID_SPEC)
    assert oracle.run(bb, 0)["rc"] == oracle.E_INVALID


def test_hpcc_compile_and_validation(simmod, oracle):
    """HPCC experiments compile onto the congestion-control kernel with a
    telemetry record per packet a window can hold; HPCC with spraying is
    rejected as the oracle rejects it."""
    b = I.make_config(11, exp_ids=[0, 7])
    s = simmod.Sim(b)
    inf = s.info()
    assert inf["n_compact"] == 0 and simmod.KERNEL_NAMES[inf["main_kernel"]] == "msim_megakernel_cc"
    assert inf["max_arena_bytes"] > simmod.Sim(I.make_config(8, exp_ids=[0, 7])).info()["max_arena_bytes"]
    for e in range(b.n_exp):
        assert s.flow_count(e) == oracle.count(b, e)[1]
    bb = I.single_batch(I.single_switch(2), I.xflows([(0, 1, 3)]), cc=I.CC_HPCC, lb=I.LB_SPRAY)
    expect_error(simmod, bb, simmod.E_INVALID_SPEC)
    assert oracle.run(bb, 0)["rc"] == oracle.E_INVALID


def test_packet_spraying_compile_and_validation(simmod, oracle):
    """Sprayed experiments compile onto the spraying kernel; unknown modes and
    spraying with congestion control are rejected as the oracle rejects them."""
    b = I.make_config(9, exp_ids=[0, 3])
    s = simmod.Sim(b)
    inf = s.info()
    assert inf["n_compact"] == 0 and simmod.KERNEL_NAMES[inf["main_kernel"]] == "msim_megakernel_sp"
    for e in range(b.n_exp):
        assert s.flow_count(e) == oracle.count(b, e)[1]
    topo = I.single_switch(2)
    w = I.xflows([(0, 1, 3)])
    for bb in (I.single_batch(topo, w, lb=2),
               I.single_batch(topo, w, lb=I.LB_SPRAY, cc=I.CC_DCTCP, ecn_k=2, cwnd0=2)):
        expect_error(simmod, bb, simmod.E_INVALID_SPEC)
        assert oracle.run(bb, 0)["rc"] == oracle.E_INVALID


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; asked for more it exits with a message (no GPU
    is touched before that check)."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_lds_probe_rejects_bad_arguments(simmod):
    """The LDS probe validates its arguments before any HIP call."""
    lib = simmod.load_library()
    E = -5   # MSIM_E_ARG
    assert lib.msim_lds_probe(None, 4096, 1, 1, None) == E          # no output buffer
    assert lib.msim_lds_probe(1, 4095, 1, 1, None) == E             # output smaller than blocks x 4 KiB
    assert lib.msim_lds_probe(1, 4096, 0, 1, None) == E             # no workgroups
    assert lib.msim_lds_probe(1, 8 << 30, (1 << 20) + 1, 1, None) == E
    assert lib.msim_lds_probe(1, 4096, 1, 0, None) == E             # no iterations


def test_bench_traffic_records(tmp_path, monkeypatch):
    """The bench line's measured HBM traffic comes from profiles/traffic.json
    only for the kernel, workload and kernel source it was taken on: a
    different kernel, config, experiment count or source text gives None."""
    import importlib
    import json
    import shutil
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    # a copy of the tree's bench, its profiles record and the kernel sources
    for d in ("profiles", os.path.join("experiment_network_simulation_amd", "csrc")):
        os.makedirs(tmp_path / d, exist_ok=True)
    shutil.copy(os.path.join(root, "bench.py"), tmp_path / "bench.py")
    for f in ("msim_kernel.hip", "msim_layout.h"):
        shutil.copy(os.path.join(root, "experiment_network_simulation_amd", "csrc", f),
                    tmp_path / "experiment_network_simulation_amd" / "csrc" / f)
    recs = json.load(open(os.path.join(root, "profiles", "traffic.json")))
    json.dump(recs, open(tmp_path / "profiles" / "traffic.json", "w"))
    monkeypatch.syspath_prepend(str(tmp_path))
    sys.modules.pop("bench", None)
    bench = importlib.import_module("bench")
    assert bench.__file__.startswith(str(tmp_path))
    import hashlib
    h = hashlib.sha256()
    for f in ("msim_kernel.hip", "msim_layout.h"):
        h.update(open(tmp_path / "experiment_network_simulation_amd" / "csrc" / f, "rb").read())
    for r in recs:
        # a record taken on an older source is simply not used
        want = r["traffic_bytes_per_launch"] if r["kernel_source_sha256"] == h.hexdigest() else None
        assert bench.measured_traffic(r["kernel"], r["config"], r["experiments"]) == want
        assert bench.measured_traffic(r["kernel"] + "_x", r["config"], r["experiments"]) is None
        assert bench.measured_traffic(r["kernel"], r["config"] + 1, r["experiments"]) is None
        assert bench.measured_traffic(r["kernel"], r["config"], r["experiments"] - 1) is None
    # any edit of the kernel source, a comment included, retires the records
    k = tmp_path / "experiment_network_simulation_amd" / "csrc" / "msim_layout.h"
    k.write_text(k.read_text() + "\n")
    for r in recs:
        assert bench.measured_traffic(r["kernel"], r["config"], r["experiments"]) is None
    sys.modules.pop("bench", None)
