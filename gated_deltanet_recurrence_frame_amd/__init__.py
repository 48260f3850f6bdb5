"""libgdn: frame-wise Gated DeltaNet token mixer on MI355X (gfx950).

The compute path is the HIP shared library ``libgdn.so`` built from
``csrc/``; ``binding`` is a thin ctypes layer over its C ABI (argument
marshalling only).  ``inputs`` draws seeded synthetic problems.
Importing the package does not load the library; the first binding call does,
and it raises if the library is missing.
"""

__all__ = ["binding", "inputs"]
