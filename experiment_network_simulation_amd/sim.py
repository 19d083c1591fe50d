"""Thin Python binding of libmsim (include/msim.h): argument marshalling only.

Every step of the simulation runs in the HIP library; PyTorch only provides the
device workspace and the stream.  There is no fallback: if libmsim.so is
missing, importing the binding fails.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsim.so")

ABI_VERSION = 5
OK, S_INCOMPLETE, S_DEADLOCK = 0, 1, 2
E_INVALID_SPEC, E_UNROUTABLE, E_WORKSPACE, E_HIP, E_ARG, E_STATE, E_LIMIT = -1, -2, -3, -4, -5, -6, -7
EXP_DONE, EXP_INCOMPLETE, EXP_DEADLOCK = 0, 1, 2
NONE = 0xFFFFFFFF

KERNEL_NAMES = ["msim_megakernel", "msim_megakernel_c8h_r1", "msim_megakernel_c8h", "msim_megakernel_c8w_r1",
                "msim_megakernel_c8w", "msim_megakernel_c16h_r1", "msim_megakernel_c16h", "msim_megakernel_c16w_r1",
                "msim_megakernel_c16w", "msim_megakernel_t", "msim_megakernel_cc", "msim_megakernel_c8h_r1_x",
                "msim_megakernel_c16h_x", "msim_megakernel_sp", "msim_megakernel_ring"]

EXPORTED = ["msim_create", "msim_workspace_size", "msim_bind", "msim_run", "msim_run_noalloc", "msim_reset",
            "msim_results",
            "msim_flow_count", "msim_flow_ticks", "msim_task_count", "msim_task_ticks", "msim_get_info",
            "msim_last_error", "msim_destroy", "msim_lds_probe"]

_P8, _P32, _P64 = C.POINTER(C.c_uint8), C.POINTER(C.c_uint32), C.POINTER(C.c_uint64)


class MsimError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"msim error {code}: {msg}")
        self.code = code


class _Spec(C.Structure):
    _fields_ = [("version", C.c_uint32), ("n_topo", C.c_uint32), ("n_work", C.c_uint32), ("n_exp", C.c_uint32),
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


class _Options(C.Structure):
    _fields_ = [("version", C.c_uint32), ("n_record", C.c_uint32), ("record_exp", _P32),
                ("host_threads", C.c_uint32), ("force_global", C.c_uint32), ("block_threads", C.c_uint32),
                ("no_ring_path", C.c_uint32), ("reserved", C.c_uint32 * 7)]


class _Info(C.Structure):
    _fields_ = [("n_exp", C.c_uint32), ("block_threads", C.c_uint32), ("grid_blocks", C.c_uint32),
                ("lds_bytes", C.c_uint32), ("n_lds_exp", C.c_uint32), ("n_compact", C.c_uint32),
                ("main_kernel", C.c_uint32), ("max_ports", C.c_uint32),
                ("max_arena_bytes", C.c_uint64), ("total_flows", C.c_uint64), ("total_conns", C.c_uint64),
                ("est_pkt_hops", C.c_uint64), ("est_delivered", C.c_uint64), ("workspace_bytes", C.c_uint64)]


_lib = None


def load_library():
    """Loads libmsim.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmsim.so not found at {LIB_PATH}; build it with "
                          "`python -m experiment_network_simulation_amd.build` (no fallback exists)")
    lib = C.CDLL(LIB_PATH)
    vp = C.c_void_p
    lib.msim_create.argtypes = [C.POINTER(_Spec), C.POINTER(_Options), C.POINTER(vp)]
    lib.msim_workspace_size.argtypes = [vp, _P64]
    lib.msim_bind.argtypes = [vp, vp, C.c_uint64, vp]
    lib.msim_run.argtypes = [vp, C.c_uint32, vp, C.c_uint32]
    lib.msim_run_noalloc.argtypes = [vp, C.c_uint32, vp, C.c_uint32]
    lib.msim_reset.argtypes = [vp, vp]
    lib.msim_results.argtypes = [vp, vp, _P8, _P32, _P64, _P64, _P64]
    lib.msim_flow_count.argtypes = [vp, C.c_uint32, _P64]
    lib.msim_flow_ticks.argtypes = [vp, C.c_uint32, vp, _P32, _P32, _P32]
    lib.msim_task_count.argtypes = [vp, C.c_uint32, _P32]
    lib.msim_task_ticks.argtypes = [vp, C.c_uint32, vp, _P32, _P32]
    lib.msim_get_info.argtypes = [vp, C.POINTER(_Info)]
    lib.msim_last_error.argtypes = [vp]
    lib.msim_last_error.restype = C.c_char_p
    lib.msim_destroy.argtypes = [vp]
    lib.msim_destroy.restype = None
    lib.msim_lds_probe.argtypes = [vp, C.c_uint64, C.c_uint32, C.c_uint32, vp]
    for name in EXPORTED:
        if name not in ("msim_last_error", "msim_destroy"):
            getattr(lib, name).restype = C.c_int
    _lib = lib
    return lib


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def lds_probe(out, blocks: int, iters: int, stream=None) -> int:
    """Launches the LDS read-bandwidth probe (msim_lds_probe) on the stream.
    `out` is a device tensor of at least blocks x 4,096 bytes.  Returns the
    bytes the launch reads from LDS; the caller times it on the same stream."""
    lib = load_library()
    nbytes = out.numel() * out.element_size()
    rc = lib.msim_lds_probe(C.c_void_p(out.data_ptr()), nbytes, blocks, iters, C.c_void_p(_stream_ptr(stream)))
    if rc != 0:
        raise MsimError(rc, "msim_lds_probe: bad arguments or launch failure")
    return blocks * 1024 * iters * 128


class Sim:
    """A compiled batch.  create -> bind(workspace) -> run -> results."""

    def __init__(self, batch, record: Sequence[int] = (), force_global: bool = False, block_threads: int = 0,
                 host_threads: int = 0, no_ring_path: bool = False):
        lib = load_library()
        p = batch.pack() if hasattr(batch, "pack") else batch
        self.packed = p
        self.n_exp = p.n_exp
        self._spec = _Spec(ABI_VERSION, p.n_topo, p.n_work, p.n_exp,
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
        self._rec = np.ascontiguousarray(np.asarray(list(record), np.uint32))
        self.record = [int(x) for x in self._rec]
        opts = _Options(ABI_VERSION, len(self._rec), _ptr(self._rec, _P32) if len(self._rec) else None,
                        host_threads, 1 if force_global else 0, block_threads, 1 if no_ring_path else 0)
        ctx = C.c_void_p()
        rc = lib.msim_create(C.byref(self._spec), C.byref(opts), C.byref(ctx))
        if rc != OK:
            raise MsimError(rc, lib.msim_last_error(None).decode())
        self._ctx = ctx
        self._lib = lib
        self.ws = None
        n = np.zeros(1, np.uint64)
        lib.msim_workspace_size(ctx, _ptr(n, _P64))
        self.workspace_bytes = int(n[0])

    def _check(self, rc: int):
        if rc < 0:
            raise MsimError(rc, self._lib.msim_last_error(self._ctx).decode())
        return rc

    def info(self) -> Dict:
        inf = _Info()
        self._check(self._lib.msim_get_info(self._ctx, C.byref(inf)))
        return {k: getattr(inf, k) for k, _ in _Info._fields_}

    def bind(self, device: str = "cuda:0", stream=None, workspace=None):
        import torch
        if workspace is None:
            workspace = torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=device)
        self.ws = workspace
        self._check(self._lib.msim_bind(self._ctx, C.c_void_p(workspace.data_ptr()),
                                        workspace.numel() * workspace.element_size(),
                                        C.c_void_p(_stream_ptr(stream))))
        return self

    def run(self, max_ticks: int = 0xFFFFFFF0, stream=None):
        self._check(self._lib.msim_run(self._ctx, max_ticks, C.c_void_p(_stream_ptr(stream)), 0))

    def run_noalloc(self, max_ticks: int = 0xFFFFFFF0, stream=None):
        """msim_run_noalloc: the same run with the queue counters in the
        library's static device array (no allocation anywhere)."""
        self._check(self._lib.msim_run_noalloc(self._ctx, max_ticks, C.c_void_p(_stream_ptr(stream)), 0))

    def reset(self, stream=None):
        self._check(self._lib.msim_reset(self._ctx, C.c_void_p(_stream_ptr(stream))))

    def results(self, stream=None) -> Dict[str, np.ndarray]:
        E = self.n_exp
        st = np.zeros(E, np.uint8)
        tk = np.zeros(E, np.uint32)
        hops, dlv, dig = (np.zeros(E, np.uint64) for _ in range(3))
        rc = self._check(self._lib.msim_results(self._ctx, C.c_void_p(_stream_ptr(stream)), _ptr(st, _P8),
                                                _ptr(tk, _P32), _ptr(hops, _P64), _ptr(dlv, _P64), _ptr(dig, _P64)))
        return dict(rc=rc, status=st, tick=tk, pkt_hops=hops, delivered=dlv, digest=dig)

    def flow_count(self, exp: int) -> int:
        n = np.zeros(1, np.uint64)
        self._check(self._lib.msim_flow_count(self._ctx, exp, _ptr(n, _P64)))
        return int(n[0])

    def flow_ticks(self, exp: int, stream=None) -> Dict[str, np.ndarray]:
        n = self.flow_count(exp)
        rd, act, sd = (np.zeros(max(n, 1), np.uint32) for _ in range(3))
        self._check(self._lib.msim_flow_ticks(self._ctx, exp, C.c_void_p(_stream_ptr(stream)), _ptr(rd, _P32),
                                              _ptr(act, _P32), _ptr(sd, _P32)))
        return dict(rd=rd[:n], act=act[:n], sd=sd[:n])

    def task_count(self, exp: int) -> int:
        n = np.zeros(1, np.uint32)
        self._check(self._lib.msim_task_count(self._ctx, exp, _ptr(n, _P32)))
        return int(n[0])

    def task_ticks(self, exp: int, stream=None) -> Dict[str, np.ndarray]:
        """Start and finish tick of every task of experiment exp (NONE if not yet)."""
        n = self.task_count(exp)
        st, fi = np.zeros(max(n, 1), np.uint32), np.zeros(max(n, 1), np.uint32)
        self._check(self._lib.msim_task_ticks(self._ctx, exp, C.c_void_p(_stream_ptr(stream)), _ptr(st, _P32),
                                              _ptr(fi, _P32)))
        return dict(start=st[:n], finish=fi[:n])

    def close(self):
        if getattr(self, "_ctx", None):
            self._lib.msim_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
