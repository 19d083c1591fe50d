"""Brute-force tick stepper: the tick contract written out as plainly as
possible, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  It shares no code with the C oracle or with the HIP
library; it reads the same generator objects (inputs.Batch) and computes
everything else itself.  It exists to pin the oracle where no closed form
reaches: round-robin and credit interplay under heavy mixing.

What it transcribes (the pages' passages the rules come from):
  - Multiverse, section 3.2 "System execution graph": the systems of one
    simulation step run in a fixed order (schedule, send, NIC send, forward,
    transmit, NIC receive);
  - Multiverse, section 4.2 "Pull-based data synchronisation": each ingress
    keeps the set of egresses it has packets for and every egress pulls;
  - Multiverse, section 5 "Implementation": one step is the smallest link delay;
    flows come from NCCL's ring algorithms; ECMP balances load;
  - AutoCCL, section 2.3 (Table 2): NC channels run concurrently, the chunks of a
    channel one after the other;
  - AlpaComm, section 3.1, Fig. 3d: a receiver forwards a partition once it
    holds all of it.
The readings of what the pages leave open (the tick rules R1-R6 and workload
rules W1-W3 of the oracle's header) are restated at each step below.

Unlike the oracle, nothing here is event-driven or precomputed: every tick
visits every port, every flow and every queue, and each round of a tick first
decides every grant on the state at the start of the round and only then
applies them.  With shuffle=<random.Random>, every phase visits its entities
in a fresh random order; the contract makes the result independent of it.
"""

from __future__ import annotations

import random
from typing import Dict, List, Optional

from experiment_network_simulation_amd import inputs as I

INF = float("inf")


def murmur_fmix32(h: int) -> int:
    """MurmurHash3's 32-bit finaliser (public domain, Austin Appleby)."""
    h &= 0xFFFFFFFF
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & 0xFFFFFFFF
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & 0xFFFFFFFF
    h ^= h >> 16
    return h


class Deadlock(Exception):
    pass


def _order(items, rng: Optional[random.Random]):
    items = list(items)
    if rng is not None:
        rng.shuffle(items)
    return items


def _ports(topo: I.Topology):
    """A node's ports in the order its cables are listed.  Each port:
    (node, neighbour, rate leaving through it, delay, alive)."""
    ports = [[] for _ in range(topo.n_nodes)]
    for c in range(topo.n_cables):
        a, b = int(topo.cable_a[c]), int(topo.cable_b[c])
        d, al = int(topo.delay[c]), bool(topo.alive[c])
        ports[a].append(dict(node=a, nbr=b, rate=int(topo.rate_ab[c]), delay=d, alive=al))
        ports[b].append(dict(node=b, nbr=a, rate=int(topo.rate_ba[c]), delay=d, alive=al))
    for n in range(topo.n_nodes):
        for k, p in enumerate(ports[n]):
            p["local"] = k
    # the port at the far end of each port
    for n in range(topo.n_nodes):
        for p in ports[n]:
            m = p["nbr"]
            same = [q for q in ports[m] if q["nbr"] == n]
            mine = [q for q in ports[n] if q["nbr"] == m]
            p["far"] = (m, same[mine.index(p)]["local"])
    return ports


def _route(topo: I.Topology, ports, src: int, dst: int, key: int, seed: int) -> List[int]:
    """Local egress port at every node from src to dst: at each node the
    candidates are the alive ports that continue a fewest-links path that only
    climbs layers and then only descends them; the connection takes
    cand[H mod |cand|], H = fmix32(key ^ fmix32(node ^ seed)), candidates in
    port order."""
    L = topo.layer
    # fewest links to dst from (node, may still climb), by relaxing until stable
    dist = {}
    for n in range(topo.n_nodes):
        for up in (True, False):
            dist[(n, up)] = 0 if n == dst else INF
    changed = True
    while changed:
        changed = False
        for n in range(topo.n_nodes):
            for up in (True, False):
                best = dist[(n, up)]
                for p in ports[n]:
                    if not p["alive"]:
                        continue
                    m = p["nbr"]
                    if L[m] > L[n] and up:
                        cand = dist[(m, True)] + 1
                    elif L[m] < L[n]:
                        cand = dist[(m, False)] + 1
                    else:
                        continue
                    if cand < best:
                        best = cand
                if best < dist[(n, up)]:
                    dist[(n, up)] = best
                    changed = True
    path, n, up = [], src, True
    while n != dst:
        need = dist[(n, up)]
        if need == INF:
            raise ValueError("unroutable")
        cands = []
        for p in ports[n]:
            if not p["alive"]:
                continue
            m = p["nbr"]
            if L[m] > L[n] and up and dist[(m, True)] + 1 == need:
                cands.append(p["local"])
            elif L[m] < L[n] and dist[(m, False)] + 1 == need:
                cands.append(p["local"])
        h = murmur_fmix32(key ^ murmur_fmix32(n ^ seed))
        k = cands[h % len(cands)]
        path.append(k)
        m = ports[n][k]["nbr"]
        if L[m] < L[n]:
            up = False
        n = m
    return path


def _flows(work: I.Workload, pkt: int):
    """Connections (src, dst) and flows (conn, size, preds) in the numbering of
    the C ABI: collectives in input order (a ring by channel, round, step,
    rank; a broadcast by hop, partition), then explicit flows.  preds: list of
    (flow, 'recv' | 'send')."""
    conns, flows = [], []
    for col in work.colls:
        m = col.members
        N = len(m)
        P = -(-col.nbytes // pkt)
        if col.kind in (I.COLL_RING_AR, I.COLL_RING_AG, I.COLL_RING_RS):
            NC, p = col.nc, col.chunk_bytes // pkt
            S = 2 * (N - 1) if col.kind == I.COLL_RING_AR else N - 1
            for c in range(NC):
                Pc = P // NC + (1 if c < P % NC else 0)
                R = -(-Pc // (N * p))
                # a last round of fewer than N packets joins the round before it
                if R > 1 and Pc - (R - 1) * N * p < N:
                    R -= 1
                c0 = len(conns)
                for i in range(N):
                    conns.append((m[i], m[(i + 1) % N]))
                base = len(flows)

                def fid(r, s, i):
                    return base + (r * S + s) * N + i
                for r in range(R):
                    X = N * p if r + 1 < R else Pc - (R - 1) * N * p
                    for s in range(S):
                        for i in range(N):
                            if col.kind == I.COLL_RING_AR and s >= N - 1:
                                k = (i + 1 - (s - (N - 1))) % N
                            else:
                                k = (i - s) % N
                            size = X // N + (1 if k < X % N else 0)
                            preds = []
                            if s >= 1:
                                preds = [(fid(r, s - 1, (i - 1) % N), "recv"), (fid(r, s - 1, i), "send")]
                            elif r >= 1:
                                preds = [(fid(r - 1, S - 1, i), "send")]
                            flows.append(dict(conn=c0 + i, size=size, preds=preds))
        elif col.kind == I.COLL_PIPE_BCAST:
            K = col.k
            c0 = len(conns)
            for j in range(1, N):
                conns.append((m[j - 1], m[j]))
            base = len(flows)
            for j in range(1, N):
                for k in range(K):
                    preds = []
                    if j >= 2:
                        preds.append((base + (j - 2) * K + k, "recv"))
                    if k >= 1:
                        preds.append((base + (j - 1) * K + k - 1, "send"))
                    size = P // K + (1 if k < P % K else 0)
                    flows.append(dict(conn=c0 + j - 1, size=size, preds=preds))
        else:
            raise ValueError("the stepper covers rings, broadcasts and explicit flows")
    for s, d, n in zip(work.xsrc, work.xdst, work.xpkts):
        conns.append((int(s), int(d)))
        flows.append(dict(conn=len(conns) - 1, size=int(n), preds=[]))
    return conns, flows


def simulate(batch: I.Batch, e: int, shuffle: Optional[random.Random] = None,
             max_ticks: int = 1_000_000) -> Dict:
    x = batch.exps[e]
    topo, work = batch.topos[x.topo], batch.works[x.work]
    Q, seed = x.queue_pkts, x.ecmp_seed
    ports = _ports(topo)
    L = topo.layer
    conns, flows = _flows(work, x.pkt_bytes)
    paths = [_route(topo, ports, s, d, ci, seed) for ci, (s, d) in enumerate(conns)]
    R = max([p["rate"] for n in range(topo.n_nodes) for p in ports[n]] + [1])
    F = len(flows)
    rd, act, sd = [None] * F, [None] * F, [None] * F
    recv, sent = [0] * F, [0] * F
    conn_flows = [[] for _ in conns]
    for f, fl in enumerate(flows):
        conn_flows[fl["conn"]].append(f)
    nic_inputs = {n: [ci for ci, (s, _) in enumerate(conns) if s == n] for n in range(topo.n_nodes)}
    # switch ingress buffers: every packet sent on the cable into the port and
    # not yet forwarded, in sending order; hosts: packets on the wire to them
    buf = {(n, k): [] for n in range(topo.n_nodes) for k in range(len(ports[n]))}
    rr = {(n, k): 0 for n in range(topo.n_nodes) for k in range(len(ports[n]))}
    hops = delivered = 0
    max_occ = 0
    t = 0
    while True:
        if t >= max_ticks:
            return dict(status="incomplete", t_end=t, rd=rd, act=act, sd=sd, pkt_hops=hops,
                        delivered=delivered, max_occupancy=max_occ)
        # A: packets reaching a host at t are delivered; a flow whose last
        # packet arrives gets RD = t
        for (n, k) in _order([q for q in buf if L[q[0]] == 0], shuffle):
            keep = []
            for pk in buf[(n, k)]:
                if pk["arrive"] == t:
                    f = pk["flow"]
                    recv[f] += 1
                    delivered += 1
                    if recv[f] == flows[f]["size"]:
                        rd[f] = t
                else:
                    keep.append(pk)
            buf[(n, k)] = keep
        # B: a flow activates at the first tick its predecessors are met
        # (RECV: RD <= t; SEND: SD <= t)
        activated = False
        for f in _order(range(F), shuffle):
            if act[f] is not None:
                continue
            ok = all((rd[g] if kind == "recv" else sd[g]) is not None and
                     (rd[g] if kind == "recv" else sd[g]) <= t for g, kind in flows[f]["preds"])
            if ok:
                act[f] = t
                activated = True
        # C: credit of every output: Q minus the packets sent into the far
        # ingress and not yet forwarded before t; no limit towards a host
        credit = {}
        for (n, k) in buf:
            p = ports[n][k]
            fn, fk = p["far"]
            credit[(n, k)] = INF if L[fn] == 0 else Q - len(buf[(fn, fk)])
        # D: rounds
        tx = False
        granted = {q: 0 for q in buf}
        for m in range(R):
            grants = []
            for (n, k) in _order(list(buf), shuffle):
                p = ports[n][k]
                if not p["alive"] or m >= p["rate"] or granted[(n, k)] >= p["rate"] or credit[(n, k)] <= 0:
                    continue
                if L[n] == 0:
                    inputs = nic_inputs[n]
                    cand = []
                    for j, ci in enumerate(inputs):
                        cur = [f for f in conn_flows[ci] if act[f] is not None and sent[f] < flows[f]["size"]]
                        if cur:
                            cand.append(j)
                else:
                    inputs = list(range(len(ports[n])))
                    cand = []
                    for i in inputs:
                        voq = [pk for pk in buf[(n, i)] if pk["egress"] == k]
                        if voq and voq[0]["arrive"] <= t:
                            cand.append(i)
                if not cand:
                    continue
                start = rr[(n, k)]
                pick = min(cand, key=lambda j: (j - start) % len(inputs))
                grants.append((n, k, pick, len(inputs)))
            for (n, k, pick, nin) in _order(grants, shuffle):
                p = ports[n][k]
                if L[n] == 0:
                    ci = nic_inputs[n][pick]
                    f = [f for f in conn_flows[ci] if act[f] is not None and sent[f] < flows[f]["size"]][0]
                    sent[f] += 1
                    if sent[f] == flows[f]["size"]:
                        sd[f] = t + 1
                    pk = dict(flow=f, conn=ci, pos=0)
                else:
                    voq = [pk for pk in buf[(n, pick)] if pk["egress"] == k]
                    pk = voq[0]
                    buf[(n, pick)].remove(pk)
                fn, fk = p["far"]
                pos = pk["pos"] + 1
                path = paths[pk["conn"]]
                nxt = dict(flow=pk["flow"], conn=pk["conn"], pos=pos, arrive=t + p["delay"],
                           egress=path[pos] if pos < len(path) else None)
                buf[(fn, fk)].append(nxt)
                if L[fn] != 0:
                    max_occ = max(max_occ, len(buf[(fn, fk)]))
                    if len(buf[(fn, fk)]) > Q:
                        raise AssertionError("buffer over capacity")
                credit[(n, k)] -= 1
                granted[(n, k)] += 1
                rr[(n, k)] = (pick + 1) % nin
                hops += 1
                tx = True
        # E: done once every flow has arrived; a tick with no sending, no
        # activation and nothing on the wire, while not done, is a deadlock
        if all(v is not None for v in rd):
            t_end = max(rd) if F else 0
            return dict(status="done", t_end=t_end, rd=rd, act=act, sd=sd, pkt_hops=hops,
                        delivered=delivered, max_occupancy=max_occ)
        on_wire = any(pk["arrive"] > t for q in buf for pk in buf[q])
        if not tx and not activated and not on_wire:
            return dict(status="deadlock", t_end=t, rd=rd, act=act, sd=sd, pkt_hops=hops,
                        delivered=delivered, max_occupancy=max_occ)
        t += 1
