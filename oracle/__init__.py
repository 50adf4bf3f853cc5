"""fp64 CPU oracle for the gated delta rule (test infrastructure only).

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg
may import this package; the library never does.
"""
from .gdr_oracle import (L2_EPS, backward, chunked_forward, forward, l2norm,
                         l2norm_vjp)

__all__ = ["L2_EPS", "forward", "backward", "chunked_forward", "l2norm",
           "l2norm_vjp"]
