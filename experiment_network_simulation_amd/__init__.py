"""Batched packet-level network simulator for AMD MI355X (gfx950).

Thousands of independent experiments -- collective-communication traffic over
switched topologies -- simulated tick by tick in one HIP megakernel behind the
C ABI of include/msim.h.  `inputs` builds seeded synthetic batches; `sim.Sim`
is the thin binding over libmsim.so.
"""

from . import inputs  # noqa: F401

__all__ = ["inputs", "Sim", "load_library"]


def __getattr__(name):
    if name in ("Sim", "load_library", "MsimError"):
        from . import sim
        return getattr(sim, name)
    raise AttributeError(name)
