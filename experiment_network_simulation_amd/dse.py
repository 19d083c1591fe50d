"""Design-space exploration over the batched simulator.

Two drivers from the pages, each scoring its candidates by simulation, all
candidates of one step in one batch (single program, many experiments):

  tune()        AutoCCL section 4.3: subspace-oriented tuning (Algorithm 1) with a
                coordinate descent over the resource parameters in each subspace
                (Algorithm 2).  Every (task, subspace) search advances in lockstep:
                each step gathers the next configuration of every search that
                needs a simulation and runs them as one batch.
  reshard()     AlpaComm section 3.2: unit-task schedules from the naive,
                load-balance-only, DFS-with-pruning and randomised greedy
                schedulers, turned into task graphs of pipelined broadcasts and
                scored in one batch.

Readings (the same as the plain reference of the test-suite):
  - A subspace is the algorithm: ring or tree for an all-reduce, ring otherwise.
    The resource parameters are NC and C, grids of values addressed by index.
  - Bandwidth is bytes / T (T: simulated completion tick).  A probe improves when
    its T is lower; the improvement fraction T_opt / T_p - 1 becomes the learning
    rate, whose step moves the current dimension up by max(1, floor(lr * grid
    length)) indices, clamped to the grid.  Without improvement the next
    dimension is taken at rate 0.01.  The first probe is the random start; a
    search stops after M + 1 probes in a row without improvement; a point
    profiled before is not simulated again.  The earlier subspace wins ties.
  - A unit task's duration for the analytical schedulers is the broadcast time
    of section 3.1 with t = P packets ticks: ceil(P (K + A - 1) / K).  A task
    starts once every earlier task in the global order that shares one of its
    hosts has finished.  Naive: lowest holder, input order.  Load balance: by
    decreasing duration to the least-loaded holder, input order.  DFS: optimal
    order and senders under that rule.  Greedy: stages of host-disjoint tasks,
    the round covering most hosts among R random visiting orders (keys given).

Random draws (descent starts, greedy keys) are inputs from the input module.
"""

from __future__ import annotations

import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import inputs as I

# ---------------------------------------------------------------------------
# Scoring a list of experiments on the GPU
# ---------------------------------------------------------------------------


@dataclass
class Probe:
    """One experiment to score: a workload on a topology."""
    topo: I.Topology
    work: I.Workload
    queue_pkts: int
    ecmp_seed: int


@dataclass
class EvalStats:
    batches: int = 0
    experiments: int = 0
    pkt_hops: int = 0
    delivered: int = 0
    kernel_ms: float = 0.0
    host_s: float = 0.0


class GpuEvaluator:
    """Scores probes with the HIP simulator, one batch per call."""

    def __init__(self, device: str = "cuda:0", max_ticks: int = 0xFFFFFFF0):
        import torch
        from .sim import Sim
        if not torch.cuda.is_available():
            raise RuntimeError("GpuEvaluator needs a GPU")
        self.torch, self.Sim = torch, Sim
        self.device, self.max_ticks = device, max_ticks
        self.stream = torch.cuda.Stream(device=device)
        self.stats = EvalStats()

    def __call__(self, probes: Sequence[Probe]) -> np.ndarray:
        if not probes:
            return np.zeros(0, np.int64)
        t0 = time.perf_counter()
        batch = make_batch(probes)
        sim = self.Sim(batch)
        torch = self.torch
        with torch.cuda.stream(self.stream):
            sim.bind(self.device, stream=self.stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            sim.run(self.max_ticks, stream=self.stream)
            b.record(self.stream)
            r = sim.results(stream=self.stream)
        self.stream.synchronize()
        if np.any(r["status"] != 0):
            bad = np.nonzero(r["status"] != 0)[0]
            raise RuntimeError(f"simulation did not complete for probes {bad[:8].tolist()}")
        self.stats.batches += 1
        self.stats.experiments += len(probes)
        self.stats.pkt_hops += int(r["pkt_hops"].sum())
        self.stats.delivered += int(r["delivered"].sum())
        self.stats.kernel_ms += a.elapsed_time(b)
        sim.close()
        self.stats.host_s += time.perf_counter() - t0
        return r["tick"].astype(np.int64)


def make_batch(probes: Sequence[Probe]) -> I.Batch:
    """One experiment per probe; topologies shared by identity."""
    topos, tmap, works, exps = [], {}, [], []
    for p in probes:
        k = id(p.topo)
        if k not in tmap:
            tmap[k] = len(topos)
            topos.append(p.topo)
        works.append(p.work)
        exps.append(I.Experiment(tmap[k], len(works) - 1, p.queue_pkts, p.ecmp_seed))
    return I.Batch(topos, works, exps, "dse")


# ---------------------------------------------------------------------------
# AutoCCL: lockstep coordinate descent
# ---------------------------------------------------------------------------


class Descent:
    """Algorithm 2 as a state machine: `want` is the point to profile next
    (None once finished); `feed(T)` supplies its completion tick."""

    def __init__(self, sizes: Sequence[int], start: Sequence[int]):
        self.sizes = tuple(int(n) for n in sizes)
        self.want: Optional[Tuple[int, ...]] = tuple(int(x) for x in start)
        self.best = self.want
        self.best_t: Optional[int] = None
        self.dim = 0
        self.misses = 0
        self.trace: List[Tuple[Tuple[int, ...], int]] = []

    def feed(self, t: int) -> None:
        p = self.want
        self.trace.append((p, t))
        gain_num, gain_den = 1, 100
        if self.best_t is not None and t < self.best_t:
            gain_num, gain_den = self.best_t - t, t
            self.best, self.best_t, self.misses = p, t, 0
        else:
            if self.best_t is None:
                self.best_t = t
            self.misses += 1
            self.dim = (self.dim + 1) % len(self.sizes)
        if self.misses > len(self.sizes):
            self.want = None
            return
        n = self.sizes[self.dim]
        q = list(self.best)
        q[self.dim] = min(q[self.dim] + max(1, gain_num * n // gain_den), n - 1)
        self.want = tuple(q)


def algorithms_for(kind: int) -> List[int]:
    return [I.COLL_RING_AR, I.COLL_TREE_AR] if kind == I.COLL_RING_AR else [kind]


@dataclass
class TuneResult:
    algo: int
    nc: int
    chunk: int
    ticks: int
    per_subspace: List[Dict] = field(default_factory=list)


def tune(tasks: Sequence[I.TuneTask], starts: np.ndarray, evaluate, nc_grid: Sequence[int] = I.TUNE_NC,
         chunk_grid: Sequence[int] = I.TUNE_CHUNK, log=None) -> List[TuneResult]:
    """Tunes every task's (algorithm, NC, C); starts[t, s] is the random start
    of task t's search in its s-th subspace.  evaluate(probes) -> ticks."""
    sizes = (len(nc_grid), len(chunk_grid))
    searches = []                        # (task, algorithm, Descent)
    for t, task in enumerate(tasks):
        for s, algo in enumerate(algorithms_for(task.kind)):
            searches.append((t, algo, Descent(sizes, starts[t, s])))
    seen: Dict[Tuple[int, int, Tuple[int, ...]], int] = {}
    step = 0
    while True:
        need: Dict[Tuple[int, int, Tuple[int, ...]], int] = {}
        for t, algo, d in searches:
            while d.want is not None and (t, algo, d.want) in seen:
                d.feed(seen[(t, algo, d.want)])
            if d.want is not None and (t, algo, d.want) not in need:
                need[(t, algo, d.want)] = len(need)
        if not need:
            break
        probes = []
        for (t, algo, p) in need:
            task = tasks[t]
            c = I.Collective(algo, task.nbytes, list(task.members), nc_grid[p[0]], chunk_grid[p[1]], 1)
            probes.append(Probe(task.topo, I.Workload([c]), task.queue_pkts, task.ecmp_seed))
        ticks = evaluate(probes)
        for key, k in need.items():
            seen[key] = int(ticks[k])
        step += 1
        if log:
            log(f"[tune] step {step}: {len(probes)} probes")
    out = []
    for t, task in enumerate(tasks):
        mine = [(algo, d) for tt, algo, d in searches if tt == t]
        k_best = 0
        for k in range(1, len(mine)):
            if mine[k][1].best_t < mine[k_best][1].best_t:
                k_best = k
        algo, d = mine[k_best]
        out.append(TuneResult(algo, nc_grid[d.best[0]], chunk_grid[d.best[1]], d.best_t,
                              [dict(algo=a, best=dd.best, ticks=dd.best_t, trace=dd.trace) for a, dd in mine]))
    return out


# ---------------------------------------------------------------------------
# AlpaComm: unit-task schedulers
# ---------------------------------------------------------------------------


@dataclass
class Schedule:
    sender: List[int]
    order: List[int]
    makespan: int                        # analytical, under the start rule
    complete: bool = True                # False: DFS stopped at its node budget


def durations(tasks: Sequence[I.UnitComm], K: int) -> List[int]:
    """Analytical duration of every task; rejects tasks whose receivers repeat
    or include a holder (a broadcast chain visits each host once)."""
    out = []
    for u in tasks:
        if not u.holders or not u.receivers or len(set(u.receivers)) != len(u.receivers) \
                or set(u.holders) & set(u.receivers):
            raise ValueError(f"invalid unit task {u}")
        P = -(-u.nbytes // I.PKT_BYTES)
        out.append(-(-P * (K + len(u.receivers) - 1) // K))
    return out


def analytic_makespan(tasks, dur, sender, order) -> int:
    ready: Dict[int, int] = {}
    end = 0
    for i in order:
        hs = (sender[i], *tasks[i].receivers)
        s = max(ready.get(h, 0) for h in hs)
        for h in hs:
            ready[h] = s + dur[i]
        end = max(end, s + dur[i])
    return end


def sched_naive(tasks, dur) -> Schedule:
    snd = [min(u.holders) for u in tasks]
    order = list(range(len(tasks)))
    return Schedule(snd, order, analytic_makespan(tasks, dur, snd, order))


def sched_load_balance(tasks, dur) -> Schedule:
    load: Dict[int, int] = {}
    snd = [0] * len(tasks)
    for i in sorted(range(len(tasks)), key=lambda i: (-dur[i], i)):
        h = min(u for u in tasks[i].holders if load.get(u, 0) == min(load.get(v, 0) for v in tasks[i].holders))
        snd[i] = h
        load[h] = load.get(h, 0) + dur[i]
    order = list(range(len(tasks)))
    return Schedule(snd, order, analytic_makespan(tasks, dur, snd, order))


def sched_greedy(tasks, dur, keys: np.ndarray) -> Schedule:
    """keys[stage, round, task]: round r of stage s visits the remaining tasks by
    (key, index)."""
    n = len(tasks)
    rec = [frozenset(u.receivers) for u in tasks]
    hold = [sorted(u.holders) for u in tasks]
    left = np.ones(n, bool)
    snd = [0] * n
    order: List[int] = []
    stage = 0
    while left.any():
        idx = np.nonzero(left)[0]
        best = None
        for r in range(keys.shape[1]):
            kk = keys[stage, r, idx]
            visit = idx[np.lexsort((idx, kk))]
            used: set = set()
            pick: List[Tuple[int, int]] = []
            for i in visit.tolist():
                if not rec[i].isdisjoint(used):
                    continue
                h = next((h for h in hold[i] if h not in used and h not in rec[i]), None)
                if h is None:
                    continue
                pick.append((i, h))
                used.update(rec[i])
                used.add(h)
            if best is None or len(used) > best[0]:
                best = (len(used), pick)
        for i, h in best[1]:
            snd[i] = h
            order.append(i)
            left[i] = False
        stage += 1
    return Schedule(snd, order, analytic_makespan(tasks, dur, snd, order))


def sched_dfs(tasks, dur, node_budget: int = 2_000_000, upper: Optional[Schedule] = None) -> Schedule:
    """Optimal schedule under the start rule.  Only orders sorted by (start,
    index) are enumerated: every schedule the rule produces is reproduced by
    that order, so nothing is lost.  Branches are cut by the largest host load
    (placed tasks on their sender and receivers, unplaced ones on their
    receivers).  Stops after node_budget nodes (complete=False)."""
    n = len(tasks)
    rec = [tuple(u.receivers) for u in tasks]
    hold = [sorted(u.holders) for u in tasks]
    hosts = sorted({h for u in tasks for h in (*u.holders, *u.receivers)})
    hid = {h: k for k, h in enumerate(hosts)}
    H = len(hosts)
    rec_load = np.zeros(H, np.int64)
    for i in range(n):
        for h in rec[i]:
            rec_load[hid[h]] += dur[i]
    best = [upper.makespan if upper is not None else None, list(upper.sender) if upper else None,
            list(upper.order) if upper else None]
    nodes = [0]
    free = np.zeros(H, np.int64)
    load = np.zeros(H, np.int64)          # placed work on the host + unplaced work it receives
    load[:] = rec_load
    snd = [0] * n
    order: List[int] = []
    placed = [False] * n

    def visit(last_s: int, last_i: int, span: int) -> bool:
        nodes[0] += 1
        if nodes[0] > node_budget:
            return False
        if len(order) == n:
            if best[0] is None or span < best[0]:
                best[0], best[1], best[2] = span, list(snd), list(order)
            return True
        if best[0] is not None and max(span, int(load.max())) >= best[0]:
            return True
        for i in range(n):
            if placed[i]:
                continue
            rs = [hid[h] for h in rec[i]]
            for h in hold[i]:
                hs = [hid[h]] + rs
                s = int(free[hs].max())
                if (s, i) < (last_s, last_i):
                    continue
                old = free[hs].copy()
                free[hs] = s + dur[i]
                load[hid[h]] += dur[i]
                placed[i] = True
                snd[i] = h
                order.append(i)
                ok = visit(s, i, max(span, s + dur[i]))
                order.pop()
                placed[i] = False
                load[hid[h]] -= dur[i]
                free[hs] = old
                if not ok:
                    return False
        return True

    done = visit(-1, -1, 0)
    return Schedule(best[1], best[2], best[0], complete=done)


def schedule_workload(tasks: Sequence[I.UnitComm], sched: Schedule, K: int) -> I.Workload:
    """Collective i: task i's pipelined broadcast from its sender along its
    receivers.  Task graph: the tasks in global order, each after the previous
    task on each of its hosts."""
    w = I.Workload([I.bcast(u.nbytes, [sched.sender[i], *u.receivers], K) for i, u in enumerate(tasks)])
    prev: Dict[int, int] = {}
    for pos, i in enumerate(sched.order):
        hs = (sched.sender[i], *tasks[i].receivers)
        w.tasks.append(I.comm(i, sorted({prev[h] for h in hs if h in prev})))
        for h in hs:
            prev[h] = pos
    return w


@dataclass
class ReshardResult:
    names: List[str]
    schedules: List[Schedule]
    simulated: np.ndarray                # completion tick of each schedule
    best: int                            # index of the lowest simulated tick (first on ties)


def reshard(instances: Sequence[Tuple[I.Topology, Sequence[I.UnitComm]]], K: int, key_sets: Sequence[np.ndarray],
            evaluate, queue_pkts: int = 16, ecmp_seed: int = 0, dfs_max_tasks: int = 0,
            dfs_budget: int = 2_000_000) -> List[ReshardResult]:
    """Every scheduler on every instance (randomised greedy once per key set;
    DFS when the instance has at most dfs_max_tasks tasks), all schedules of all
    instances scored in one batch."""
    plans = []
    for topo, tasks in instances:
        dur = durations(tasks, K)
        names = ["naive", "load_balance"]
        scheds = [sched_naive(tasks, dur), sched_load_balance(tasks, dur)]
        for g, keys in enumerate(key_sets):
            names.append(f"greedy{g}")
            scheds.append(sched_greedy(tasks, dur, keys))
        if len(tasks) <= dfs_max_tasks:
            names.append("dfs")
            scheds.append(sched_dfs(tasks, dur, dfs_budget))
        plans.append((topo, tasks, names, scheds))
    probes = [Probe(topo, schedule_workload(tasks, s, K), queue_pkts, ecmp_seed)
              for topo, tasks, _, scheds in plans for s in scheds]
    ticks = evaluate(probes)
    out, k = [], 0
    for topo, tasks, names, scheds in plans:
        t = ticks[k:k + len(scheds)]
        k += len(scheds)
        out.append(ReshardResult(names, scheds, t, int(np.argmin(t))))
    return out
