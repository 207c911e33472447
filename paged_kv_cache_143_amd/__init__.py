"""Paged decode attention for MI355X (gfx950).

The compute path lives in the HIP library `libpa.so` (sources in `csrc/`,
C-ABI in `include/pa.h`); `binding` is its thin ctypes binding, `blocks` the
host-side block manager that produces block tables, slots and copy-on-write
pairs, and `workloads` the seeded synthetic inputs.  Importing the package
loads nothing; `binding.lib()` loads the library and fails loudly when it is
missing.
"""
__all__ = ["binding", "blocks", "workloads"]
