"""CPU oracle for the DSV block-sparse attention path -- test infrastructure only.

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``; the HIP library never imports or calls it.
"""
from . import dsv_oracle  # noqa: F401
