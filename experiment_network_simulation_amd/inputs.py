"""Seeded synthetic inputs for the batched packet simulator.

This module draws and lays out the *inputs* of a batch of independent network
experiments: switched topologies (nodes, cables, rates, delays, dead cables),
collective workloads (ring all-reduce / ring all-gather described by message
size, channel count NC and chunk size C; K-partition pipelined broadcast; sparse
explicit flows) and per-experiment parameters (queue depth, ECMP seed, packet
size).  It performs none of the simulator's own arithmetic: it does not turn
bytes into packets, split messages into channels/rounds/chunks, compute routes
or simulate anything.  Both the HIP library and the CPU oracle consume exactly
the arrays built here and derive everything else independently.

The experiment shapes follow the pages:
  * the usage model (Multiverse, section 3.1 "Architecture": the user sets
    topology, workload and CCL parameters and lists the experiments to run),
  * NCCL's channel count NC and chunk size C (AutoCCL, section 2.3, Table 2),
  * the K-partition pipelined broadcast (AlpaComm, section 3.1, Fig. 3d),
  * sparse variable-volume rank-to-rank traffic (Perplexity MoE blog, the
    expert-parallel + data-parallel discussion).

Random draws use SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; the public-domain reference
constants of Vigna's splitmix64.c).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# Node layers: hosts are layer 0; switches 1 (edge/leaf), 2 (agg/spine), 3 (core).
LAYER_HOST = 0

# Collective kinds (values are part of the C ABI and of the oracle's input).
COLL_RING_AR = 1
COLL_RING_AG = 2
COLL_PIPE_BCAST = 3
COLL_RING_RS = 4        # ring reduce-scatter (message = total input)
COLL_TREE_AR = 5        # binary-tree all-reduce, pipelined in chunks
COLL_SENDRECV = 6       # one source sends the whole message to each receiver in turn
NO_GATE = 0xFFFFFFFF

# Task kinds of a workload's task graph (values are part of the C ABI).
TASK_COMPUTE = 0        # a computation of `ticks` ticks
TASK_INTRA = 1          # an intra-server collective: alpha + ceil(bytes / beta) ticks
TASK_COLL = 2           # a collective of the workload, simulated packet by packet

CC_NONE = 0             # congestion control of an experiment
CC_DCTCP = 1            # ECN marking at switches, ACKs, DCTCP windows per connection
CC_DCQCN = 2            # ECN marking at switches, CNPs, DCQCN rates per connection
CC_HPCC = 3             # in-band telemetry at switch egresses, ACKs, HPCC windows per connection

LB_ECMP = 0             # load balancing of an experiment: one route per connection
LB_SPRAY = 1            # every packet chooses among the equal-cost egresses at every switch

KIB = 1024
MIB = 1024 * 1024
PKT_BYTES = 4096

_M64 = (1 << 64) - 1


class SplitMix64:
    """SplitMix64 generator (public-domain reference algorithm)."""

    def __init__(self, seed: int):
        self.state = seed & _M64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & _M64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        return z ^ (z >> 31)

    def below(self, n: int) -> int:
        """Integer in [0, n) (plain modulo reduction; n is tiny here)."""
        return self.next() % n

    def between(self, lo: int, hi: int) -> int:
        """Integer in the inclusive range [lo, hi]."""
        return lo + self.below(hi - lo + 1)

    def u32(self) -> int:
        return self.next() & 0xFFFFFFFF

    def permutation(self, n: int) -> List[int]:
        """Fisher-Yates shuffle of range(n), drawn from the high index down."""
        a = list(range(n))
        for i in range(n - 1, 0, -1):
            j = self.below(i + 1)
            a[i], a[j] = a[j], a[i]
        return a


def exp_rng(base: int, e: int) -> SplitMix64:
    """Per-experiment stream: seeded with one SplitMix64 output of base ^ e."""
    return SplitMix64(SplitMix64(base ^ e).next())


# ---------------------------------------------------------------------------
# Topologies
# ---------------------------------------------------------------------------

@dataclass
class Topology:
    """Nodes (by layer) and cables.  A node's ports are numbered by the order in
    which its cables appear here; rate_ab is the packets/tick from cable_a to
    cable_b, delay the ticks per traversal (both directions)."""
    layer: np.ndarray          # uint8 [n_nodes]
    cable_a: np.ndarray        # uint32 [n_cables]
    cable_b: np.ndarray        # uint32
    rate_ab: np.ndarray        # uint8
    rate_ba: np.ndarray        # uint8
    delay: np.ndarray          # uint8
    alive: np.ndarray          # uint8
    name: str = ""

    @property
    def n_nodes(self) -> int:
        return int(self.layer.shape[0])

    @property
    def n_cables(self) -> int:
        return int(self.cable_a.shape[0])

    def hosts(self) -> np.ndarray:
        return np.nonzero(self.layer == LAYER_HOST)[0].astype(np.uint32)

    def copy(self, name: Optional[str] = None) -> "Topology":
        return Topology(self.layer.copy(), self.cable_a.copy(), self.cable_b.copy(),
                        self.rate_ab.copy(), self.rate_ba.copy(), self.delay.copy(),
                        self.alive.copy(), name if name is not None else self.name)


def topology_from_cables(layers: Sequence[int], cables: Sequence[tuple], name: str = "") -> Topology:
    """cables: (a, b[, rate_ab, rate_ba, delay, alive]) tuples, defaults 1,1,1,1."""
    a, b, rab, rba, d, al = [], [], [], [], [], []
    for c in cables:
        c = tuple(c) + (1, 1, 1, 1)[len(c) - 2:]
        a.append(c[0]); b.append(c[1]); rab.append(c[2]); rba.append(c[3]); d.append(c[4]); al.append(c[5])
    return Topology(np.asarray(layers, np.uint8), np.asarray(a, np.uint32), np.asarray(b, np.uint32),
                    np.asarray(rab, np.uint8), np.asarray(rba, np.uint8), np.asarray(d, np.uint8),
                    np.asarray(al, np.uint8), name)


def single_switch(n_hosts: int, rate: int = 1, delay: int = 1) -> Topology:
    """Hosts 0..n-1 on one switch (node n); switch port i faces host i."""
    layers = [LAYER_HOST] * n_hosts + [1]
    cables = [(h, n_hosts, rate, rate, delay, 1) for h in range(n_hosts)]
    return topology_from_cables(layers, cables, f"switch{n_hosts}")


def leaf_spine(n_leaf: int, hosts_per_leaf: int, n_spine: int, host_rate: int = 1,
               up_rate: int = 2, delay: int = 1) -> Topology:
    """Hosts first (host = leaf*hosts_per_leaf + i), then leaves, then spines.
    Leaf ports 0..hpl-1 face its hosts, then spines 0..n_spine-1; spine port l
    faces leaf l."""
    H = n_leaf * hosts_per_leaf
    leaf0, spine0 = H, H + n_leaf
    layers = [LAYER_HOST] * H + [1] * n_leaf + [2] * n_spine
    cables = []
    for h in range(H):
        cables.append((h, leaf0 + h // hosts_per_leaf, host_rate, host_rate, delay, 1))
    for l in range(n_leaf):
        for s in range(n_spine):
            cables.append((leaf0 + l, spine0 + s, up_rate, up_rate, delay, 1))
    return topology_from_cables(layers, cables, f"leafspine{n_leaf}x{hosts_per_leaf}+{n_spine}")


def fat_tree(k: int, rate: int = 1, delay: int = 1, oversub: int = 1) -> Topology:
    """k-ary fat-tree: k pods of k/2 edge switches, each edge switch serving k/2
    hosts (host id = pod*k^2/4 + edge*k/2 + i).  With oversubscription o each pod
    keeps a = k/(2o) aggregation switches, every edge switch links to all of
    them (k/2 host ports, a uplinks: o:1 at the edge layer) and aggregation
    switch j of every pod links to the k/2 core switches of group j.  o = 1 is
    the standard fat-tree.  Ports: edge 0..k/2-1 hosts, then aggs; agg 0..k/2-1
    edges, then cores; core port = pod.  Node order: hosts, edges, aggs, cores."""
    h2 = k // 2
    na = h2 // oversub
    H = k * h2 * h2
    edge0 = H
    agg0 = edge0 + k * h2
    core0 = agg0 + k * na
    layers = [LAYER_HOST] * H + [1] * (k * h2) + [2] * (k * na) + [3] * (na * h2)
    cables = []
    for h in range(H):
        cables.append((h, edge0 + h // h2, rate, rate, delay, 1))
    for p in range(k):
        for e in range(h2):
            for a in range(na):
                cables.append((edge0 + p * h2 + e, agg0 + p * na + a, rate, rate, delay, 1))
    for p in range(k):
        for a in range(na):
            for j in range(h2):
                cables.append((agg0 + p * na + a, core0 + a * h2 + j, rate, rate, delay, 1))
    return topology_from_cables(layers, cables, f"fattree{k}o{oversub}")


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclass
class Collective:
    kind: int                  # one of the COLL_* kinds
    nbytes: int                # message size (all-gather: total output; reduce-scatter: total
                               # input; send/recv: bytes each receiver gets)
    members: List[int]         # ring order; broadcast chain or send/recv (source first);
                               # tree in heap order (member 0 the root)
    nc: int = 1                # channels (rings, trees)
    chunk_bytes: int = 0       # chunk size C (rings, trees)
    k: int = 1                 # partitions (broadcast)
    gate: int = NO_GATE        # rings: index, within the workload, of an earlier send/recv
                               # whose receivers are these members; each rank then starts
                               # once its piece from that send/recv has arrived


@dataclass
class Task:
    """A node of the workload's task graph: it starts once every predecessor
    (an index of an earlier task) has finished."""
    kind: int
    ticks: int = 0             # compute: duration; intra-server: alpha (ticks)
    nbytes: int = 0            # intra-server: message bytes
    beta: int = 1              # intra-server: bytes per tick
    coll: int = -1             # collective task: index of the collective in the workload
    preds: List[int] = field(default_factory=list)


def compute(ticks: int, preds: Sequence[int] = ()) -> Task:
    return Task(TASK_COMPUTE, int(ticks), preds=[int(p) for p in preds])


def intra(alpha: int, nbytes: int, beta: int, preds: Sequence[int] = ()) -> Task:
    return Task(TASK_INTRA, int(alpha), int(nbytes), int(beta), preds=[int(p) for p in preds])


def comm(coll: int, preds: Sequence[int] = ()) -> Task:
    return Task(TASK_COLL, coll=int(coll), preds=[int(p) for p in preds])


@dataclass
class Workload:
    colls: List[Collective] = field(default_factory=list)
    xsrc: np.ndarray = field(default_factory=lambda: np.zeros(0, np.uint32))
    xdst: np.ndarray = field(default_factory=lambda: np.zeros(0, np.uint32))
    xpkts: np.ndarray = field(default_factory=lambda: np.zeros(0, np.uint32))
    tasks: List[Task] = field(default_factory=list)


def ring(kind: int, nbytes: int, members: Sequence[int], nc: int, chunk_bytes: int) -> Collective:
    return Collective(kind, int(nbytes), [int(m) for m in members], int(nc), int(chunk_bytes), 1)


def bcast(nbytes: int, chain: Sequence[int], k: int) -> Collective:
    return Collective(COLL_PIPE_BCAST, int(nbytes), [int(m) for m in chain], 1, 0, int(k))


def tree(nbytes: int, members: Sequence[int], nc: int, chunk_bytes: int) -> Collective:
    return Collective(COLL_TREE_AR, int(nbytes), [int(m) for m in members], int(nc), int(chunk_bytes), 1)


def sendrecv(nbytes_each: int, source: int, receivers: Sequence[int]) -> Collective:
    return Collective(COLL_SENDRECV, int(nbytes_each), [int(source)] + [int(m) for m in receivers], 1, 0, 1)


def unit_task(strategy: str, nbytes: int, source: int, nodes: Sequence[Sequence[int]],
              chunk_bytes: int = 0, first_index: int = 0) -> List[Collective]:
    """A unit communication task: one slice of nbytes from `source` to every
    device of A receiving nodes of B devices each (AlpaComm section 3.1,
    Figure 3), as collectives of this simulator:
      "sendrecv"  the source sends the whole slice to each device in turn;
      "local_ag"  it sends a 1/B part to each device (the nodes then assemble
                  the slice over their intra-node links, which this network
                  model does not carry);
      "global_ag" it sends a 1/(A B) part to each device, then the devices run
                  a ring all-gather of the whole slice, each one starting when
                  its part has arrived (chunk_bytes: the ring's chunk);
      "broadcast" a pipelined broadcast along the devices (use bcast).
    first_index: where the returned collectives start in their workload (the
    all-gather's gate names the send/recv by that index)."""
    devs = [int(d) for node in nodes for d in node]
    A, B = len(nodes), len(nodes[0])
    if strategy == "sendrecv":
        return [sendrecv(nbytes, source, devs)]
    if strategy == "local_ag":
        return [sendrecv(nbytes // B, source, devs)]
    if strategy == "global_ag":
        part = sendrecv(nbytes // (A * B), source, devs)
        ag = ring(COLL_RING_AG, nbytes, devs, 1, chunk_bytes)
        ag.gate = int(first_index)
        return [part, ag]
    raise ValueError(strategy)


def xflows(pairs: Sequence[tuple]) -> Workload:
    """Explicit flows (src, dst, packets), kept in the given order."""
    w = Workload()
    if pairs:
        arr = np.asarray(pairs, dtype=np.int64)
        w.xsrc, w.xdst, w.xpkts = (arr[:, 0].astype(np.uint32), arr[:, 1].astype(np.uint32),
                                   arr[:, 2].astype(np.uint32))
    return w


# ---------------------------------------------------------------------------
# Batch
# ---------------------------------------------------------------------------

@dataclass
class Experiment:
    topo: int
    work: int
    queue_pkts: int
    ecmp_seed: int
    pkt_bytes: int = PKT_BYTES
    cc: int = CC_NONE          # CC_NONE, CC_DCTCP, CC_DCQCN or CC_HPCC
    ecn_k: int = 0             # DCTCP, DCQCN: marking threshold (packets)
    cwnd0: int = 0             # DCTCP: initial window (packets, >= 1)
    lb: int = LB_ECMP          # LB_ECMP or LB_SPRAY


@dataclass
class Batch:
    """A batch of experiments referencing shared topologies and workloads."""
    topos: List[Topology]
    works: List[Workload]
    exps: List[Experiment]
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def n_exp(self) -> int:
        return len(self.exps)

    def subset(self, idx: Sequence[int]) -> "Batch":
        """The listed experiments, with only the topologies/workloads they use."""
        idx = list(idx)
        tmap, wmap, topos, works, exps = {}, {}, [], [], []
        for i in idx:
            x = self.exps[i]
            if x.topo not in tmap:
                tmap[x.topo] = len(topos); topos.append(self.topos[x.topo])
            if x.work not in wmap:
                wmap[x.work] = len(works); works.append(self.works[x.work])
            exps.append(Experiment(tmap[x.topo], wmap[x.work], x.queue_pkts, x.ecmp_seed, x.pkt_bytes,
                                   x.cc, x.ecn_k, x.cwnd0, x.lb))
        meta = dict(self.meta)
        meta["subset_of"] = self.name
        meta["subset_idx"] = idx
        return Batch(topos, works, exps, self.name, meta)

    def pack(self) -> "PackedBatch":
        return PackedBatch.from_batch(self)


@dataclass
class PackedBatch:
    """Flat CSR arrays in the exact layout both consumers read."""
    n_topo: int
    n_work: int
    n_exp: int
    topo_node_off: np.ndarray    # uint32 [n_topo+1]
    node_layer: np.ndarray       # uint8
    topo_cable_off: np.ndarray   # uint32 [n_topo+1]
    cable_a: np.ndarray          # uint32 (node index local to its topology)
    cable_b: np.ndarray
    cable_rate_ab: np.ndarray    # uint8
    cable_rate_ba: np.ndarray
    cable_delay: np.ndarray
    cable_alive: np.ndarray
    work_coll_off: np.ndarray    # uint32 [n_work+1]
    coll_type: np.ndarray        # uint8
    coll_bytes: np.ndarray       # uint64
    coll_nc: np.ndarray          # uint32
    coll_chunk_bytes: np.ndarray # uint32
    coll_k: np.ndarray           # uint32
    coll_member_off: np.ndarray  # uint32 [n_coll+1]
    member_host: np.ndarray      # uint32
    coll_gate: np.ndarray        # uint32 (NO_GATE, or a collective index within the workload)
    work_task_off: np.ndarray    # uint32 [n_work+1]
    task_type: np.ndarray        # uint8
    task_ticks: np.ndarray       # uint32
    task_bytes: np.ndarray       # uint64
    task_beta: np.ndarray        # uint32
    task_coll: np.ndarray        # uint32
    task_pred_off: np.ndarray    # uint32 [n_task+1]
    task_pred: np.ndarray        # uint32 (task indices within the workload)
    work_xflow_off: np.ndarray   # uint64 [n_work+1]
    xflow_src: np.ndarray        # uint32
    xflow_dst: np.ndarray
    xflow_pkts: np.ndarray
    exp_topo: np.ndarray         # uint32 [n_exp]
    exp_work: np.ndarray
    exp_queue_pkts: np.ndarray
    exp_ecmp_seed: np.ndarray
    exp_pkt_bytes: np.ndarray
    exp_cc: np.ndarray           # uint8
    exp_ecn_k: np.ndarray        # uint32
    exp_cwnd0: np.ndarray        # uint32
    exp_lb: np.ndarray           # uint8

    @staticmethod
    def from_batch(b: Batch) -> "PackedBatch":
        def cat(xs, dt):
            return np.ascontiguousarray(np.concatenate(xs).astype(dt)) if xs else np.zeros(0, dt)

        t_node_off = np.zeros(len(b.topos) + 1, np.uint32)
        t_cab_off = np.zeros(len(b.topos) + 1, np.uint32)
        for i, t in enumerate(b.topos):
            t_node_off[i + 1] = t_node_off[i] + t.n_nodes
            t_cab_off[i + 1] = t_cab_off[i] + t.n_cables
        colls = [c for w in b.works for c in w.colls]
        w_coll_off = np.zeros(len(b.works) + 1, np.uint32)
        w_x_off = np.zeros(len(b.works) + 1, np.uint64)
        for i, w in enumerate(b.works):
            w_coll_off[i + 1] = w_coll_off[i] + len(w.colls)
            w_x_off[i + 1] = w_x_off[i] + len(w.xsrc)
        m_off = np.zeros(len(colls) + 1, np.uint32)
        for i, c in enumerate(colls):
            m_off[i + 1] = m_off[i] + len(c.members)
        tasks = [k for w in b.works for k in w.tasks]
        w_task_off = np.zeros(len(b.works) + 1, np.uint32)
        for i, w in enumerate(b.works):
            w_task_off[i + 1] = w_task_off[i] + len(w.tasks)
        p_off = np.zeros(len(tasks) + 1, np.uint32)
        for i, k in enumerate(tasks):
            p_off[i + 1] = p_off[i] + len(k.preds)
        return PackedBatch(
            n_topo=len(b.topos), n_work=len(b.works), n_exp=len(b.exps),
            topo_node_off=t_node_off,
            node_layer=cat([t.layer for t in b.topos], np.uint8),
            topo_cable_off=t_cab_off,
            cable_a=cat([t.cable_a for t in b.topos], np.uint32),
            cable_b=cat([t.cable_b for t in b.topos], np.uint32),
            cable_rate_ab=cat([t.rate_ab for t in b.topos], np.uint8),
            cable_rate_ba=cat([t.rate_ba for t in b.topos], np.uint8),
            cable_delay=cat([t.delay for t in b.topos], np.uint8),
            cable_alive=cat([t.alive for t in b.topos], np.uint8),
            work_coll_off=w_coll_off,
            coll_type=np.asarray([c.kind for c in colls], np.uint8),
            coll_bytes=np.asarray([c.nbytes for c in colls], np.uint64),
            coll_nc=np.asarray([c.nc for c in colls], np.uint32),
            coll_chunk_bytes=np.asarray([c.chunk_bytes for c in colls], np.uint32),
            coll_k=np.asarray([c.k for c in colls], np.uint32),
            coll_member_off=m_off,
            member_host=np.asarray([m for c in colls for m in c.members], np.uint32),
            coll_gate=np.asarray([c.gate for c in colls], np.uint32),
            work_task_off=w_task_off,
            task_type=np.asarray([k.kind for k in tasks], np.uint8),
            task_ticks=np.asarray([k.ticks for k in tasks], np.uint32),
            task_bytes=np.asarray([k.nbytes for k in tasks], np.uint64),
            task_beta=np.asarray([k.beta for k in tasks], np.uint32),
            task_coll=np.asarray([k.coll & 0xFFFFFFFF for k in tasks], np.uint32),
            task_pred_off=p_off,
            task_pred=np.asarray([q for k in tasks for q in k.preds], np.uint32),
            work_xflow_off=w_x_off,
            xflow_src=cat([w.xsrc for w in b.works], np.uint32),
            xflow_dst=cat([w.xdst for w in b.works], np.uint32),
            xflow_pkts=cat([w.xpkts for w in b.works], np.uint32),
            exp_topo=np.asarray([x.topo for x in b.exps], np.uint32),
            exp_work=np.asarray([x.work for x in b.exps], np.uint32),
            exp_queue_pkts=np.asarray([x.queue_pkts for x in b.exps], np.uint32),
            exp_ecmp_seed=np.asarray([x.ecmp_seed & 0xFFFFFFFF for x in b.exps], np.uint32),
            exp_pkt_bytes=np.asarray([x.pkt_bytes for x in b.exps], np.uint32),
            exp_cc=np.asarray([x.cc for x in b.exps], np.uint8),
            exp_ecn_k=np.asarray([x.ecn_k for x in b.exps], np.uint32),
            exp_cwnd0=np.asarray([x.cwnd0 for x in b.exps], np.uint32),
            exp_lb=np.asarray([x.lb for x in b.exps], np.uint8),
        )


def single_batch(topo: Topology, work: Workload, queue_pkts: int = 16, ecmp_seed: int = 0,
                 pkt_bytes: int = PKT_BYTES, name: str = "custom", cc: int = CC_NONE, ecn_k: int = 0,
                 cwnd0: int = 0, lb: int = LB_ECMP) -> Batch:
    return Batch([topo], [work], [Experiment(0, 0, queue_pkts, ecmp_seed, pkt_bytes, cc, ecn_k, cwnd0, lb)], name)


# ---------------------------------------------------------------------------
# The five benchmark configurations
# ---------------------------------------------------------------------------

BASE_SEED = {1: 0xC1, 2: 0xC2, 3: 0xC3, 4: 0xC4, 5: 0xC5, 6: 0xC6, 7: 0xC7, 8: 0xC8, 9: 0xC9, 10: 0xCA, 11: 0xCB}
FULL_E = {1: 16, 2: 256, 3: 1024, 4: 4096, 5: 10000, 6: 768, 7: 256, 8: 256, 9: 256, 10: 256, 11: 256}
CONFIG_NAMES = {
    1: "C1 ring all-reduce 1 MiB, 8 hosts on one switch, NC x C grid",
    2: "C2 ring all-reduce 64 MiB over a 4x8 leaf-spine with 4 spines",
    3: "C3 pipelined broadcast 64 MiB to A hosts, K partitions, random delays",
    4: "C4 k=8 fat-tree: 16 DP ring all-reduces 256 MiB + 16 TP ring all-gathers 56 MiB",
    5: "C5 k=16 fat-tree sweep: Zipf(1.1) sparse all-to-all, 8 MiB per host",
    6: "C6 k=8 fat-tree collectives mix: tree all-reduces, ring reduce-scatters, send/recv unit tasks",
    7: "C7 k=8 fat-tree training iteration: compute, intra-server TP collectives, bucketed DP ring all-reduces",
    8: "C8 k=8 fat-tree with DCTCP: C4's groups and failures at a quarter of the bytes, ECN threshold and "
       "initial window swept",
    9: "C9 k=8 fat-tree with packet spraying: C4's groups and failures at a quarter of the bytes",
    10: "C10 k=8 fat-tree with DCQCN: C4's groups and failures at a quarter of the bytes, ECN threshold swept",
    11: "C11 k=8 fat-tree with HPCC: C4's groups and failures at a quarter of the bytes",
}


def _c1(e_list):
    topo = single_switch(8, 1, 1)
    works, exps = [], []
    ncs, chunks = [1, 2, 4, 8], [16, 32, 64, 128]
    for e in e_list:
        nc, ck = ncs[(e // 4) % 4], chunks[e % 4]
        works.append(Workload([ring(COLL_RING_AR, 1 * MIB, range(8), nc, ck * KIB)]))
        exps.append(Experiment(0, len(works) - 1, 16, 0))
    return Batch([topo], works, exps, "C1")


def _c2(e_list):
    topo = leaf_spine(4, 8, 4, host_rate=1, up_rate=2, delay=1)
    works, exps = [], []
    for e in e_list:
        g = exp_rng(BASE_SEED[2], e)
        nc = g.between(1, 16)
        ck = 4 * KIB * g.between(8, 128)
        seed = g.u32()
        works.append(Workload([ring(COLL_RING_AR, 64 * MIB, range(32), nc, ck)]))
        exps.append(Experiment(0, len(works) - 1, 32, seed))
    return Batch([topo], works, exps, "C2")


_C3_A = [2, 4, 8, 16]
_C3_K = [1, 2, 4, 8, 16, 32, 64]


def _c3(e_list):
    base = leaf_spine(4, 8, 4, host_rate=1, up_rate=2, delay=1)
    topos, works, exps = [], [], []
    for e in e_list:
        g = exp_rng(BASE_SEED[3], e)
        cell = e % 28
        A, K = _C3_A[cell // 7], _C3_K[cell % 7]
        t = base.copy(f"leafspine-c3-e{e}")
        t.delay = np.asarray([g.between(1, 4) for _ in range(t.n_cables)], np.uint8)
        perm = g.permutation(32)
        seed = g.u32()
        topos.append(t)
        works.append(Workload([bcast(64 * MIB, perm[:A + 1], K)]))
        exps.append(Experiment(len(topos) - 1, len(works) - 1, 32, seed))
    return Batch(topos, works, exps, "C3")


def fat_tree_reachable(k: int, alive_ea: np.ndarray, alive_ac: np.ndarray) -> bool:
    """True if every pair of edge switches of a k-ary fat-tree is joined by an
    up-then-down path.  alive_ea[p, e, a]: edge e - agg a cable of pod p alive;
    alive_ac[p, a, j]: agg a of pod p - core a*(k/2)+j alive.  Input feasibility
    check for the failure draw (edge switch pairs cover every host pair)."""
    # cp[p1, p2, a]: some core of group a is alive towards both pods.
    cp = np.einsum("paj,qaj->pqa", alive_ac.astype(np.int64), alive_ac.astype(np.int64)) > 0
    same_pod = np.eye(k, dtype=bool)[:, :, None]
    link = cp | same_pod                                     # [p1, p2, a]
    ea = alive_ea.astype(bool)                               # [p, e, a]
    # reach[p1, e1, p2, e2] = any_a ea[p1,e1,a] & ea[p2,e2,a] & link[p1,p2,a]
    reach = np.einsum("pea,qfa,pqa->peqf", ea.astype(np.int64), ea.astype(np.int64),
                      link.astype(np.int64)) > 0
    h2 = k // 2
    eye = np.zeros((k, h2, k, h2), bool)
    for p in range(k):
        for e in range(h2):
            eye[p, e, p, e] = True
    return bool(np.all(reach | eye))


def _c4_groups():
    tp = [[8 * t + i for i in range(8)] for t in range(16)]
    dp = [[g + 16 * j for j in range(8)] for g in range(16)]
    return dp, tp


def _c4(e_list):
    k = 8
    base = fat_tree(k, 1, 1)
    h2 = k // 2
    H = k * h2 * h2
    n_host_cables = H
    n_ea = k * h2 * h2
    dp, tp = _c4_groups()
    topos, works, exps = [], [], []
    for e in e_list:
        g = exp_rng(BASE_SEED[4], e)
        pi = g.permutation(H)
        nc = g.between(1, 16)
        ck = 4 * KIB * g.between(8, 128)
        nfail = g.between(0, 4)
        while True:
            pool = list(range(n_host_cables, base.n_cables))   # the 256 switch-to-switch cables
            dead = []
            for _ in range(nfail):
                j = g.below(len(pool))
                dead.append(pool.pop(j))
            alive = np.ones(base.n_cables, np.uint8)
            alive[dead] = 0
            sw = alive[n_host_cables:]
            a_ea = sw[:n_ea].reshape(k, h2, h2)
            a_ac = sw[n_ea:].reshape(k, h2, h2)
            if fat_tree_reachable(k, a_ea, a_ac):
                break
        seed = g.u32()
        t = base.copy(f"fattree8-e{e}")
        t.alive = alive
        topos.append(t)
        colls = [ring(COLL_RING_AR, 256 * MIB, [pi[r] for r in grp], nc, ck) for grp in dp]
        colls += [ring(COLL_RING_AG, 56 * MIB, [pi[r] for r in grp], nc, ck) for grp in tp]
        works.append(Workload(colls))
        exps.append(Experiment(len(topos) - 1, len(works) - 1, 16, seed))
    return Batch(topos, works, exps, "C4")


def zipf_alltoall(n_hosts: int, pkts_per_src: int, s: float, seed: int) -> Workload:
    """Per source, a seeded permutation ranks the other hosts; rank j (1-based)
    gets weight j^-s; weights are scaled to pkts_per_src packets by largest
    remainder (ties to the lower rank); zero-packet pairs carry no flow.  Flows
    are listed by source, then destination id."""
    g = SplitMix64(seed)
    j = np.arange(1, n_hosts, dtype=np.float64)
    w = j ** (-s)
    q = pkts_per_src * w / w.sum()
    base = np.floor(q).astype(np.int64)
    rem = pkts_per_src - int(base.sum())
    frac = q - base
    order = np.argsort(-frac, kind="stable")
    cnt = base.copy()
    cnt[order[:rem]] += 1
    src, dst, pk = [], [], []
    for h in range(n_hosts):
        others = [x for x in range(n_hosts) if x != h]
        perm = g.permutation(n_hosts - 1)
        per_dst = np.zeros(n_hosts, np.int64)
        for rank, pi in enumerate(perm):
            per_dst[others[pi]] = cnt[rank]
        nz = np.nonzero(per_dst)[0]
        src.append(np.full(nz.shape, h)); dst.append(nz); pk.append(per_dst[nz])
    wl = Workload()
    wl.xsrc = np.concatenate(src).astype(np.uint32)
    wl.xdst = np.concatenate(dst).astype(np.uint32)
    wl.xpkts = np.concatenate(pk).astype(np.uint32)
    return wl


def _c5(e_list, k: int = 16):
    topos = [fat_tree(k, 1, 1, o) for o in (1, 2, 4)]
    H = k * (k // 2) ** 2
    work = zipf_alltoall(H, (8 * MIB) // PKT_BYTES, 1.1, BASE_SEED[5])
    exps = []
    for e in e_list:
        g = exp_rng(BASE_SEED[5], e)
        oi = g.below(3)
        q = g.between(16, 128)
        seed = g.u32()
        exps.append(Experiment(oi, 0, q, seed))
    return Batch(topos, [work], exps, "C5")


def _c6(e_list):
    """The further collective shapes on C4's fabric (k=8 fat-tree, rate 1,
    delay 1, Q = 16, no failures), hosts placed by a seeded permutation pi of
    the 128 ranks.  Experiment e carries, by e mod 3:
      0  eight binary-tree all-reduces of 64 MiB over ranks 16g .. 16g+15,
         NC ~ U{1..4}, chunk ~ 4 KiB U{8..64} (one draw for all eight);
      1  sixteen ring reduce-scatters of 56 MiB over ranks 8t .. 8t+7 (the TP
         groups of C4), NC ~ U{1..8}, chunk ~ 4 KiB U{8..128};
      2  eight unit tasks: source rank g sends an 8 MiB slice to two nodes of
         four devices (ranks 8 + 8g .. 8 + 8g + 7), strategy by (e div 3) mod 3
         in send/recv, local all-gather, global all-gather (ring chunk
         ~ 4 KiB U{1..16})."""
    topo = fat_tree(8, 1, 1)
    H = topo.hosts().size
    works, exps = [], []
    strategies = ["sendrecv", "local_ag", "global_ag"]
    for e in e_list:
        g = exp_rng(BASE_SEED[6], e)
        pi = g.permutation(H)
        v = e % 3
        colls = []
        if v == 0:
            nc, ck = g.between(1, 4), 4 * KIB * g.between(8, 64)
            colls = [tree(64 * MIB, [pi[r] for r in range(16 * j, 16 * j + 16)], nc, ck) for j in range(8)]
        elif v == 1:
            nc, ck = g.between(1, 8), 4 * KIB * g.between(8, 128)
            colls = [ring(COLL_RING_RS, 56 * MIB, [pi[r] for r in range(8 * j, 8 * j + 8)], nc, ck)
                     for j in range(16)]
        else:
            strat = strategies[(e // 3) % 3]
            ck = 4 * KIB * g.between(1, 16)
            for j in range(8):
                base = 8 + 8 * j
                nodes = [[pi[base + 4 * a + i] for i in range(4)] for a in range(2)]
                colls += unit_task(strat, 8 * MIB, pi[j], nodes, chunk_bytes=ck, first_index=len(colls))
        works.append(Workload(colls))
        exps.append(Experiment(0, len(works) - 1, 16, g.u32()))
    return Batch([topo], works, exps, "C6")


# A tick is one 4 KiB packet on a rate-1 link; at 400 Gb/s that is about 82 ns,
# in which a 900 GB/s intra-server link moves about 72 KiB.
INTRA_BYTES_PER_TICK = 72 * KIB


def training_iteration(pi: Sequence[int], layers: int, fwd: int, bwd: int, buckets: int, nc: int, chunk: int,
                       tp_bytes: int = 56 * MIB, dp_bytes: int = 256 * MIB, alpha: int = 50) -> Workload:
    """One training iteration as a task graph (the System Simulator's input).
    Each of the 128 hosts is a server whose GPUs form one tensor-parallel
    group, so TP collectives are intra-server (the analytical model); data
    parallelism runs across servers in 16 ring groups of 8, group g being the
    servers pi[g], pi[g+16], .., pi[g+112] (C4's DP groups).
      forward:  per layer, compute(fwd) then an intra-server TP all-gather of
                tp_bytes (alpha + bytes / INTRA_BYTES_PER_TICK ticks);
      backward: per layer, compute(bwd) then an intra-server TP reduce-scatter;
      DP:       the gradients of dp_bytes per DP group in `buckets` buckets;
                bucket j (layers in reverse order) starts on each of the 16 DP
                rings once the backward layer that completes it is done;
      step:     an optimizer compute of fwd ticks after the last bucket."""
    tasks: List[Task] = []
    colls: List[Collective] = []
    prev = []
    for _ in range(layers):
        tasks.append(compute(fwd, prev)); k = len(tasks) - 1
        tasks.append(intra(alpha, tp_bytes, INTRA_BYTES_PER_TICK, [k])); prev = [len(tasks) - 1]
    per_bucket = max(1, layers // buckets)
    dp_groups = [[pi[g + 16 * j] for j in range(8)] for g in range(16)]
    bucket_tasks: List[int] = []
    for l in range(layers):
        tasks.append(compute(bwd, prev)); k = len(tasks) - 1
        tasks.append(intra(alpha, tp_bytes, INTRA_BYTES_PER_TICK, [k])); prev = [len(tasks) - 1]
        if (l + 1) % per_bucket == 0 or l == layers - 1:
            for grp in dp_groups:
                colls.append(ring(COLL_RING_AR, dp_bytes // buckets, grp, nc, chunk))
                tasks.append(comm(len(colls) - 1, [k]))
                bucket_tasks.append(len(tasks) - 1)
    tasks.append(compute(fwd, prev + bucket_tasks))
    w = Workload(colls)
    w.tasks = tasks
    return w


def _c7(e_list):
    """Training iterations on C4's fabric (k=8 fat-tree, rate 1, delay 1,
    Q = 16, no failures): 8 layers, per-layer forward compute ~ U{1000..4000}
    ticks and backward twice that, DP buckets ~ {1, 2, 4, 8}, NC ~ U{1..8},
    C ~ 4 KiB U{8..128}, a seeded placement pi of the 128 ranks.  The compute
    durations and the intra-server model's parameters are synthetic: the pages
    calibrate theirs on hardware and print none."""
    topo = fat_tree(8, 1, 1)
    works, exps = [], []
    for e in e_list:
        g = exp_rng(BASE_SEED[7], e)
        pi = g.permutation(128)
        fwd = g.between(1000, 4000)
        buckets = [1, 2, 4, 8][g.below(4)]
        nc, ck = g.between(1, 8), 4 * KIB * g.between(8, 128)
        works.append(training_iteration(pi, 8, fwd, 2 * fwd, buckets, nc, ck))
        exps.append(Experiment(0, len(works) - 1, 16, g.u32()))
    return Batch([topo], works, exps, "C7")


def _c8(e_list):
    """C4's experiments (same placements, NC, C, failed cables and ECMP seeds)
    with every message a quarter of C4's (64 MiB all-reduces, 14 MiB
    all-gathers) and DCTCP: ECN threshold K ~ U{2..16} packets and initial
    window W0 ~ U{8..64} packets, drawn from a stream of their own."""
    b = _c4(e_list)
    for w in b.works:
        for c in w.colls:
            c.nbytes //= 4
    for x, e in zip(b.exps, e_list):
        g = exp_rng(BASE_SEED[8], e)
        x.cc, x.ecn_k, x.cwnd0 = CC_DCTCP, g.between(2, 16), g.between(8, 64)
    b.name = "C8"
    return b


def _c9(e_list):
    """C4's experiments with every message a quarter of C4's (as in C8) and
    every packet sprayed over the equal-cost paths instead of ECMP."""
    b = _c4(e_list)
    for w in b.works:
        for c in w.colls:
            c.nbytes //= 4
    for x in b.exps:
        x.lb = LB_SPRAY
    b.name = "C9"
    return b


def _c10(e_list):
    """C4's experiments with every message a quarter of C4's (as in C8) and
    DCQCN: ECN threshold K ~ U{2..16} packets, drawn from a stream of its own."""
    b = _c4(e_list)
    for w in b.works:
        for c in w.colls:
            c.nbytes //= 4
    for x, e in zip(b.exps, e_list):
        x.cc, x.ecn_k = CC_DCQCN, exp_rng(BASE_SEED[10], e).between(2, 16)
    b.name = "C10"
    return b


def _c11(e_list):
    """C4's experiments with every message a quarter of C4's (as in C8) and
    HPCC, which has no per-experiment parameter."""
    b = _c4(e_list)
    for w in b.works:
        for c in w.colls:
            c.nbytes //= 4
    for x in b.exps:
        x.cc = CC_HPCC
    b.name = "C11"
    return b


def make_config(cid: int, n_exp: Optional[int] = None, exp_ids: Optional[Sequence[int]] = None) -> Batch:
    """Batch for benchmark configuration cid (1..9).  Experiment e of a config is
    the same whatever subset is drawn, so exp_ids picks a sample of the full
    batch and n_exp the first n experiments."""
    if exp_ids is None:
        exp_ids = range(FULL_E[cid] if n_exp is None else n_exp)
    e_list = list(exp_ids)
    b = {1: _c1, 2: _c2, 3: _c3, 4: _c4, 5: _c5, 6: _c6, 7: _c7, 8: _c8, 9: _c9, 10: _c10, 11: _c11}[cid](e_list)
    b.meta["config"] = cid
    b.meta["exp_ids"] = e_list
    return b


# ---------------------------------------------------------------------------
# Inputs of the design-space-exploration drivers
# ---------------------------------------------------------------------------

# Resource-parameter grids of the collective tuner: channels NC and chunk size C
# (AutoCCL section 4.2 tunes NC, NT and C; a packet network has no thread count).
TUNE_NC = list(range(1, 17))
TUNE_CHUNK = [32 * KIB * j for j in range(1, 17)]          # 32 KiB .. 512 KiB


@dataclass
class TuneTask:
    """One communication task to tune: a collective of `kind` (ring all-reduce,
    all-gather or reduce-scatter) of nbytes over members, on a topology with the
    experiment's queue capacity and ECMP seed."""
    topo: Topology
    kind: int
    nbytes: int
    members: List[int]
    queue_pkts: int
    ecmp_seed: int


def tune_starts(seed: int, n_tasks: int, n_subspaces: int = 2,
                dims: Sequence[int] = (len(TUNE_NC), len(TUNE_CHUNK))) -> np.ndarray:
    """The random starting point of every (task, subspace) search, as grid
    indices [n_tasks, n_subspaces, len(dims)], from one SplitMix64 stream per
    task."""
    out = np.zeros((n_tasks, n_subspaces, len(dims)), np.int64)
    for t in range(n_tasks):
        g = exp_rng(seed, t)
        for s in range(n_subspaces):
            for d, n in enumerate(dims):
                out[t, s, d] = g.below(n)
    return out


def tune_tasks_c2(n: int, seed: int = 0xA7C) -> List[TuneTask]:
    """n tuning tasks on C2's leaf-spine (4 leaves x 8 hosts, 4 spines, host
    links rate 1, uplinks rate 2, delay 1, Q = 32): a 64 MiB all-reduce over
    the 32 hosts in a seeded ring order, with a seeded ECMP seed."""
    topo = leaf_spine(4, 8, 4, host_rate=1, up_rate=2, delay=1)
    out = []
    for t in range(n):
        g = exp_rng(seed ^ 0x5EED, t)
        out.append(TuneTask(topo, COLL_RING_AR, 64 * MIB, g.permutation(32), 32, g.u32()))
    return out


@dataclass
class UnitComm:
    """A unit communication task of a cross-mesh resharding (AlpaComm section
    3.2): a data slice of nbytes held by each host in `holders`, needed by every
    host in `receivers` (in broadcast-chain order)."""
    holders: List[int]
    receivers: List[int]
    nbytes: int


def resharding_tasks(seed: int, n_tasks: int, mesh_a: Sequence[int], mesh_b: Sequence[int],
                     max_holders: int = 3, max_receivers: int = 4,
                     pkts_choices: Sequence[int] = (64, 128, 256, 512)) -> List[UnitComm]:
    """n_tasks unit tasks: holders drawn from mesh_a (1..max_holders hosts),
    receivers from mesh_b (1..max_receivers hosts), slice sizes from
    pkts_choices packets; one SplitMix64 stream."""
    g = exp_rng(seed, 0x7A5C)
    out = []
    for _ in range(n_tasks):
        pa, pb = g.permutation(len(mesh_a)), g.permutation(len(mesh_b))
        nh, nr = g.between(1, max_holders), g.between(1, max_receivers)
        out.append(UnitComm([int(mesh_a[i]) for i in pa[:nh]], [int(mesh_b[i]) for i in pb[:nr]],
                            int(pkts_choices[g.below(len(pkts_choices))]) * PKT_BYTES))
    return out


def greedy_keys(seed: int, n_tasks: int, n_rounds: int, n_stages: Optional[int] = None) -> np.ndarray:
    """Random sort keys [n_stages, n_rounds, n_tasks] (u64) for the randomised
    greedy scheduler: round r of stage s visits the remaining tasks in order of
    (key, index)."""
    n_stages = n_tasks if n_stages is None else n_stages
    g = SplitMix64(seed)
    out = np.zeros((n_stages, n_rounds, n_tasks), np.uint64)
    flat = out.reshape(-1)
    for i in range(flat.size):
        flat[i] = g.next()
    return out
