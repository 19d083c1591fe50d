"""The ring kernel (msim_megakernel_ring: rings only, rate-1 links, switches of
at most 8 ports, buffers of at most 16 packets) against the oracle, flow by
flow.

Every run is bounded by a tick budget a little above the oracle's completion
tick, so a wrong kernel ends with INCOMPLETE rather than running on."""

import random

import numpy as np
import pytest

from experiment_network_simulation_amd import inputs as I

pytestmark = pytest.mark.gpu

PKT = I.PKT_BYTES


def ring_batch(seed, n_exp):
    """Random experiments the ring format takes: rings (all-reduce, all-gather,
    reduce-scatter) of 2..8 ranks and 1..4 channels, several per host, on one
    8-port switch or k=4 / k=8 fat-trees with failed cables; delays 1..4;
    buffers 1..16; uneven channel, round and chunk splits."""
    rng = random.Random(seed)
    topos, works, exps = [], [], []
    for e in range(n_exp):
        kind = e % 3
        if kind == 0:
            topo = I.single_switch(8, 1, rng.randint(1, 4))
            hosts = list(range(8))
        elif kind == 1:
            topo = I.fat_tree(4)
            topo.delay = np.array([rng.randint(1, 3) for _ in range(topo.n_cables)], np.uint8)
            hosts = list(range(16))
        else:
            b4 = I.make_config(4, exp_ids=[rng.randrange(4096)])
            topo = b4.topos[b4.exps[0].topo]
            hosts = list(range(128))
        colls = []
        for _ in range(rng.randint(1, 4)):
            N = rng.randint(2, min(8, len(hosts)))
            NC = rng.randint(1, 4)
            p = rng.randint(1, 6)
            P = NC * (N * p * rng.randint(1, 3) + rng.randint(0, N)) + rng.randint(0, NC) + NC * N
            members = rng.sample(hosts, N)
            colls.append(I.ring(rng.choice([I.COLL_RING_AR, I.COLL_RING_AG, I.COLL_RING_RS]), P * PKT,
                                members, NC, p * PKT))
        topos.append(topo)
        works.append(I.Workload(colls))
        exps.append(I.Experiment(len(topos) - 1, len(works) - 1, rng.randint(1, 16), rng.getrandbits(32)))
    return I.Batch(topos, works, exps, "ring")


def check(batch, oracle, sim, exps_with_flows):
    r = sim.results()
    for e in range(batch.n_exp):
        o = oracle.run(batch, e)
        assert o["rc"] == 0
        got = (int(r["status"][e]), int(r["tick"][e]), int(r["pkt_hops"][e]), int(r["delivered"][e]),
               int(r["digest"][e]))
        want = (o["status"], o["t_end"], o["pkt_hops"], o["delivered"], o["digest"])
        assert got == want, f"experiment {e}: gpu {got} oracle {want}"
    for e in exps_with_flows:
        o = oracle.run(batch, e, flows=True)
        f = sim.flow_ticks(e)
        for k in ("rd", "act", "sd"):
            assert (f[k] == o[k]).all(), (e, k)


@pytest.mark.parametrize("seed", [1, 2])
def test_ring_kernel_matches_oracle(oracle, seed):
    import torch
    from experiment_network_simulation_amd.sim import KERNEL_NAMES, Sim
    torch.cuda.set_device(0)
    batch = ring_batch(seed, 12)
    budget = max(oracle.run(batch, e)["t_end"] for e in range(batch.n_exp)) + 64
    print(f"ring kernel: seed {seed}, {batch.n_exp} experiments, budget {budget} ticks", flush=True)
    sim = Sim(batch, record=list(range(batch.n_exp))).bind("cuda:0")
    assert KERNEL_NAMES[sim.info()["main_kernel"]] == "msim_megakernel_ring"
    assert sim.info()["n_compact"] == batch.n_exp
    sim.run(max_ticks=budget)
    check(batch, oracle, sim, range(batch.n_exp))


def test_ring_kernel_resumes(oracle):
    """Short runs of 37 ticks continue where the last one stopped: the state
    kept in registers and LDS between runs is saved and restored."""
    import torch
    from experiment_network_simulation_amd.sim import Sim
    torch.cuda.set_device(0)
    batch = ring_batch(7, 6)
    budget = max(oracle.run(batch, e)["t_end"] for e in range(batch.n_exp)) + 64
    sim = Sim(batch, record=[0, 4]).bind("cuda:0")
    for _ in range(budget // 37 + 2):
        sim.run(max_ticks=37)
    check(batch, oracle, sim, [0, 4])


def test_ring_kernel_c4_experiments(oracle):
    """Three C4 experiments (one NC = 16) with every flow's ticks."""
    import torch
    from experiment_network_simulation_amd.sim import KERNEL_NAMES, Sim
    torch.cuda.set_device(0)
    full = I.make_config(4, exp_ids=range(64))
    nc = [full.works[x.work].colls[0].nc for x in full.exps]
    ids = [nc.index(max(nc)), 5, 40]
    batch = I.make_config(4, exp_ids=ids)
    budget = max(oracle.run(batch, e)["t_end"] for e in range(batch.n_exp)) + 300
    sim = Sim(batch, record=list(range(batch.n_exp))).bind("cuda:0")
    assert KERNEL_NAMES[sim.info()["main_kernel"]] == "msim_megakernel_ring"
    sim.run(max_ticks=budget)
    check(batch, oracle, sim, range(batch.n_exp))
