"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 (NumPy) statement of what the paged
decode path computes, written from the pages and sharing no code with the
HIP library.  Only `tests/`, `__graft_entry__.smoke()` and `bench.py`'s CPU
baseline leg may import it; the product path never does.

Modules
  paging     address translation and slot/waste arithmetic
             ("Inside vLLM and TGI", section "Block addresses and
             fragmentation arithmetic")
  allocator  block manager with shared, reference-counted blocks and
             copy-on-write of a shared partial last block
             ("Inside vLLM and TGI", section "Exact CPU block manager and
             copy-on-write"; transcript paragraphs 3-4)
  pool       the paged K/V store the kernels read: token writes by slot and
             whole-block copies (same sources)
  attention  single-query softmax attention read through a block table, and
             its split-context form (transcript paragraph 3: the kernel reads
             through the table and token order stays correct)

Every function is pinned by `-m "not gpu"` tests against values the pages
print, closed forms, special cases, brute force or library routines; see the
docstring of each test module for which pin covers which function.
"""
