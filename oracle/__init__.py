"""Float64 CPU oracle of the frame-wise GDN recurrence.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.
"""

from .gdn_oracle import (  # noqa: F401
    backward,
    composite_forward,
    default_key_scale,
    forward,
    frame_terms,
    prologue,
    prologue_backward,
    step,
    tokenspace_forward,
)
