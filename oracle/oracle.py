"""Python access to the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test-suite, by the smoke check and by
the benchmark's CPU-baseline leg, never by the simulator package.  The oracle
reads the same generator arrays as the HIP library and computes everything
else on its own.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from typing import Dict, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# the mutation tests point this at a copy of the oracle with a planted mistake
OVERRIDE = os.environ.get("MSIM_ORACLE_LIB")
if OVERRIDE:
    LIB = OVERRIDE

OK, S_INCOMPLETE, S_DEADLOCK = 0, 1, 2
E_INVALID, E_UNROUTABLE, E_NOMEM, E_INVARIANT = -1, -2, -3, -4
NONE = 0xFFFFFFFF


def build(force: bool = True) -> str:
    """Compiles oracle.c into liboracle.so (plain gcc, -O2)."""
    if OVERRIDE:
        return LIB
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter",
                               "-shared", "-fPIC", SRC, "-o", tmp])
        os.replace(tmp, LIB)
    return LIB


_P8, _P32, _P64 = C.POINTER(C.c_uint8), C.POINTER(C.c_uint32), C.POINTER(C.c_uint64)


class _Batch(C.Structure):
    _fields_ = [("n_topo", C.c_uint32), ("n_work", C.c_uint32), ("n_exp", C.c_uint32), ("pad", C.c_uint32),
                ("topo_node_off", _P32), ("node_layer", _P8), ("topo_cable_off", _P32),
                ("cable_a", _P32), ("cable_b", _P32),
                ("cable_rate_ab", _P8), ("cable_rate_ba", _P8), ("cable_delay", _P8), ("cable_alive", _P8),
                ("work_coll_off", _P32), ("coll_type", _P8), ("coll_bytes", _P64),
                ("coll_nc", _P32), ("coll_chunk_bytes", _P32), ("coll_k", _P32),
                ("coll_member_off", _P32), ("member_host", _P32),
                ("work_xflow_off", _P64), ("xflow_src", _P32), ("xflow_dst", _P32), ("xflow_pkts", _P32),
                ("exp_topo", _P32), ("exp_work", _P32), ("exp_queue_pkts", _P32),
                ("exp_ecmp_seed", _P32), ("exp_pkt_bytes", _P32), ("coll_gate", _P32),
                ("work_task_off", _P32), ("task_type", _P8), ("task_ticks", _P32), ("task_bytes", _P64),
                ("task_beta", _P32), ("task_coll", _P32), ("task_pred_off", _P32), ("task_pred", _P32),
                ("exp_cc", _P8), ("exp_ecn_k", _P32), ("exp_cwnd0", _P32), ("exp_lb", _P8)]


class _Result(C.Structure):
    _fields_ = [("status", C.c_int32), ("t_end", C.c_uint32), ("pkt_hops", C.c_uint64),
                ("delivered", C.c_uint64), ("digest", C.c_uint64), ("n_flows", C.c_uint64),
                ("n_conns", C.c_uint64), ("max_occupancy", C.c_uint32), ("pad", C.c_uint32)]


_lib = None
_lock = threading.Lock()


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB):
                build(force=True)
            lib = C.CDLL(LIB)
            lib.orc_run.argtypes = [C.POINTER(_Batch), C.c_uint32, C.c_uint32, C.c_uint32,
                                    C.POINTER(_Result), _P32, _P32, _P32, _P32, _P32]
            lib.orc_run.restype = C.c_int
            lib.orc_count.argtypes = [C.POINTER(_Batch), C.c_uint32, _P64, _P64]
            lib.orc_count.restype = C.c_int
            lib.orc_paths.argtypes = [C.POINTER(_Batch), C.c_uint32, _P32, _P32, _P32, _P32, C.c_uint32]
            lib.orc_paths.restype = C.c_int
            lib.orc_flows.argtypes = [C.POINTER(_Batch), C.c_uint32, _P32, _P32]
            lib.orc_flows.restype = C.c_int
            lib.orc_qcn_script.argtypes = [C.c_uint32, _P32, C.POINTER(C.c_uint8), _P32]
            lib.orc_qcn_script.restype = C.c_int
            lib.orc_hpcc_script.argtypes = [C.c_uint32, C.c_uint32, C.c_uint32, _P32, _P32, _P32]
            lib.orc_hpcc_script.restype = C.c_int
            lib.orc_fmix32.argtypes = [C.c_uint32]
            lib.orc_fmix32.restype = C.c_uint32
            lib.orc_mix64.argtypes = [C.c_uint64]
            lib.orc_mix64.restype = C.c_uint64
            _lib = lib
    return _lib


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class OracleBatch:
    """Keeps the packed arrays alive while the C side points at them."""

    def __init__(self, packed):
        self.p = packed
        p = packed
        self.s = _Batch(p.n_topo, p.n_work, p.n_exp, 0,
                        _ptr(p.topo_node_off, _P32), _ptr(p.node_layer, _P8), _ptr(p.topo_cable_off, _P32),
                        _ptr(p.cable_a, _P32), _ptr(p.cable_b, _P32),
                        _ptr(p.cable_rate_ab, _P8), _ptr(p.cable_rate_ba, _P8), _ptr(p.cable_delay, _P8),
                        _ptr(p.cable_alive, _P8),
                        _ptr(p.work_coll_off, _P32), _ptr(p.coll_type, _P8), _ptr(p.coll_bytes, _P64),
                        _ptr(p.coll_nc, _P32), _ptr(p.coll_chunk_bytes, _P32), _ptr(p.coll_k, _P32),
                        _ptr(p.coll_member_off, _P32), _ptr(p.member_host, _P32),
                        _ptr(p.work_xflow_off, _P64), _ptr(p.xflow_src, _P32), _ptr(p.xflow_dst, _P32),
                        _ptr(p.xflow_pkts, _P32),
                        _ptr(p.exp_topo, _P32), _ptr(p.exp_work, _P32), _ptr(p.exp_queue_pkts, _P32),
                        _ptr(p.exp_ecmp_seed, _P32), _ptr(p.exp_pkt_bytes, _P32),
                        _ptr(p.coll_gate, _P32),
                        _ptr(p.work_task_off, _P32), _ptr(p.task_type, _P8), _ptr(p.task_ticks, _P32),
                        _ptr(p.task_bytes, _P64), _ptr(p.task_beta, _P32), _ptr(p.task_coll, _P32),
                        _ptr(p.task_pred_off, _P32), _ptr(p.task_pred, _P32),
                        _ptr(p.exp_cc, _P8), _ptr(p.exp_ecn_k, _P32), _ptr(p.exp_cwnd0, _P32),
                        _ptr(p.exp_lb, _P8))


def _as_oracle_batch(b) -> OracleBatch:
    if isinstance(b, OracleBatch):
        return b
    if hasattr(b, "pack"):
        b = b.pack()
    return OracleBatch(b)


def count(batch, e: int):
    ob = _as_oracle_batch(batch)
    nf, nc = np.zeros(1, np.uint64), np.zeros(1, np.uint64)
    rc = _load().orc_count(C.byref(ob.s), e, _ptr(nf, _P64), _ptr(nc, _P64))
    return rc, int(nf[0]), int(nc[0])


def run(batch, e: int, max_ticks: int = 0xFFFFFFFF, check: bool = False,
        flows: bool = False) -> Dict:
    """Runs experiment e.  Returns a dict with status, t_end, pkt_hops,
    delivered, digest, n_flows, n_conns, max_occupancy, rc and, with flows=True,
    per-flow arrays rd, act, sd and per-task arrays task_start, task_finish
    (NONE where the event did not happen)."""
    ob = _as_oracle_batch(batch)
    lib = _load()
    out: Dict = {}
    rd = act = sd = ts = tf = None
    if flows:
        rc, nf, _ = count(ob, e)
        if rc:
            return {"rc": rc}
        rd, act, sd = (np.full(max(nf, 1), NONE, np.uint32) for _ in range(3))
        w = int(ob.p.exp_work[e])
        nt = int(ob.p.work_task_off[w + 1] - ob.p.work_task_off[w])
        ts, tf = (np.full(max(nt, 1), NONE, np.uint32) for _ in range(2))
    res = _Result()
    rc = lib.orc_run(C.byref(ob.s), e, max_ticks, 1 if check else 0, C.byref(res),
                     _ptr(rd, _P32) if flows else None, _ptr(act, _P32) if flows else None,
                     _ptr(sd, _P32) if flows else None, _ptr(ts, _P32) if flows else None,
                     _ptr(tf, _P32) if flows else None)
    out["rc"] = rc
    if rc:
        return out
    out.update(status=res.status, t_end=res.t_end, pkt_hops=res.pkt_hops, delivered=res.delivered,
               digest=res.digest, n_flows=res.n_flows, n_conns=res.n_conns,
               max_occupancy=res.max_occupancy)
    if flows:
        out["rd"], out["act"], out["sd"] = rd[:res.n_flows], act[:res.n_flows], sd[:res.n_flows]
        out["task_start"], out["task_finish"] = ts[:nt], tf[:nt]
    return out


def paths(batch, e: int, max_len: int = 16):
    """Per connection: src host, dst host, number of links, global port index
    left from at each path position (NONE-padded)."""
    ob = _as_oracle_batch(batch)
    rc, nf, nc = count(ob, e)
    if rc:
        return rc, None
    src, dst, links = (np.zeros(max(nc, 1), np.uint32) for _ in range(3))
    pp = np.full((max(nc, 1), max_len), NONE, np.uint32)
    rc = _load().orc_paths(C.byref(ob.s), e, _ptr(src, _P32), _ptr(dst, _P32), _ptr(links, _P32),
                           _ptr(pp, _P32), max_len)
    return rc, dict(src=src[:nc], dst=dst[:nc], links=links[:nc], ports=pp[:nc])


def flows(batch, e: int):
    """Per flow: connection index and size in packets."""
    ob = _as_oracle_batch(batch)
    rc, nf, nc = count(ob, e)
    if rc:
        return rc, None
    conn, size = np.zeros(max(nf, 1), np.uint32), np.zeros(max(nf, 1), np.uint32)
    rc = _load().orc_flows(C.byref(ob.s), e, _ptr(conn, _P32), _ptr(size, _P32))
    return rc, dict(conn=conn[:nf], size=size[:nf])


def fmix32(h: int) -> int:
    return int(_load().orc_fmix32(h & 0xFFFFFFFF))


def qcn_script(events):
    """events: (tick, 'cnp' | 'send') in tick order, applied to one fresh
    DCQCN connection.  Returns one (RC, RT, alpha, next allowed tick) per
    event."""
    n = len(events)
    tick = np.array([t for t, _ in events], np.uint32)
    what = np.array([{"cnp": 0, "send": 1}[w] for _, w in events], np.uint8)
    state = np.zeros(4 * max(n, 1), np.uint32)
    rc = _load().orc_qcn_script(n, tick.ctypes.data_as(_P32), what.ctypes.data_as(C.POINTER(C.c_uint8)),
                                state.ctypes.data_as(_P32))
    if rc != 0:
        raise ValueError(f"orc_qcn_script: {rc}")
    return [tuple(int(v) for v in state[4 * i:4 * i + 4]) for i in range(n)]


def hpcc_script(T, acks):
    """acks: (sent, [(tick, packets sent, backlog, rate) per switch]) in order,
    applied to one fresh HPCC connection with base round trip T.  Returns one
    (U, W, Wc, stage) per ACK."""
    n = len(acks)
    nsw = len(acks[0][1]) if n else 1
    sent = np.array([a[0] for a in acks], np.uint32)
    rows = []
    for _, hops in acks:
        assert len(hops) == nsw
        rows.extend([h[k] for k in range(4) for h in hops])
    tel = np.array(rows, np.uint32)
    state = np.zeros(4 * max(n, 1), np.uint32)
    rc = _load().orc_hpcc_script(T, nsw, n, sent.ctypes.data_as(_P32), tel.ctypes.data_as(_P32),
                                 state.ctypes.data_as(_P32))
    if rc != 0:
        raise ValueError(f"orc_hpcc_script: {rc}")
    return [tuple(int(v) for v in state[4 * i:4 * i + 4]) for i in range(n)]


def mix64(z: int) -> int:
    return int(_load().orc_mix64(z & ((1 << 64) - 1)))
