"""msim_run_noalloc (the entry point for callers that cannot allocate) against
msim_run: identical per-experiment results and per-flow ticks, on two calls in
a row (the second on a smaller batch), and when run in short resumed pieces."""

import numpy as np
import pytest

from experiment_network_simulation_amd import inputs as I

pytestmark = pytest.mark.gpu

KEYS = ("status", "tick", "pkt_hops", "delivered", "digest")


def mixed_batch(n_c3):
    """C1's 16 rings (one kernel kind) plus C3 broadcasts (another kind), so a
    call makes more than one launch and each takes its own counter."""
    b = I.make_config(1)
    extra = I.make_config(3, exp_ids=list(range(n_c3)))
    for x in extra.exps:
        b.topos.append(extra.topos[x.topo])
        b.works.append(extra.works[x.work])
        b.exps.append(I.Experiment(len(b.topos) - 1, len(b.works) - 1, x.queue_pkts, x.ecmp_seed))
    return b


def outcome(sim):
    r = sim.results()
    return {k: np.array(r[k]) for k in KEYS}, sim.flow_ticks(0)


@pytest.mark.parametrize("n_c3", [6, 2])
def test_noalloc_matches_run(n_c3):
    import torch
    from experiment_network_simulation_amd.sim import Sim
    torch.cuda.set_device(0)
    batch = mixed_batch(n_c3)
    print(f"noalloc: {batch.n_exp} experiments", flush=True)
    ref = Sim(batch, record=[0]).bind("cuda:0")
    ref.run()
    want, want_f = outcome(ref)
    assert (want["status"] == 0).all()
    # two calls in a row on fresh contexts, the second on a smaller batch
    for sub in (list(range(batch.n_exp)), list(range(0, batch.n_exp, 3))):
        got_sim = Sim(batch.subset(sub), record=[0]).bind("cuda:0")
        got_sim.run_noalloc()
        got, got_f = outcome(got_sim)
        for k in KEYS:
            assert (got[k] == want[k][sub]).all(), k
        if sub[0] == 0:
            for k in ("rd", "act", "sd"):
                assert (got_f[k] == want_f[k]).all()


def test_noalloc_resumes_like_one_run():
    import torch
    from experiment_network_simulation_amd.sim import Sim
    torch.cuda.set_device(0)
    batch = mixed_batch(3)
    ref = Sim(batch, record=[0]).bind("cuda:0")
    ref.run()
    want, want_f = outcome(ref)
    sim = Sim(batch, record=[0]).bind("cuda:0")
    for _ in range(200):
        sim.run_noalloc(max_ticks=997)
        r = sim.results()
        if (r["status"] == 0).all():
            break
    got, got_f = outcome(sim)
    for k in KEYS:
        assert (got[k] == want[k]).all(), k
    for k in ("rd", "act", "sd"):
        assert (got_f[k] == want_f[k]).all()
