"""CPU oracle for chunk-swizzled AllGather-GEMM, GEMM-ReduceScatter and AG-MoE.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the C-ABI library under
``tile_level_communication_amd/`` and its Python binding) imports, links or
calls this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  It shares no code with the HIP path:
the two meet only in the seeded input arrays of ``seeded_inputs``.

What it is: plain, slow, obviously correct float64 (for floating point) and
integer (for plans and routing) implementations written from the pages on
tile-level communication:

* ``oracle.plan``  -- tile execution order of the communication-aware tile
  scheduler (DITRON paper notes, §3.2 "distributed swizzling"; Triton-Distributed
  talk, sections on swizzling and on non-perfect tiling; AutoOverlap §5.2
  (dependency resolution) and §5.4 with Fig. 6; Syncopate wiki, core method 5 "tile order follows chunk
  arrival").
* ``oracle.gemm``  -- AllGather-GEMM C = concat_c(A_c) @ B and GEMM-ReduceScatter
  out_r = sum_s P_s[rows of r] (DITRON §2/§4.1 workload definitions; talk,
  GEMM-ReduceScatter example).
* ``oracle.moe``   -- top-k softmax routing, per-expert row lists ordered by
  chunk arrival, grouped GEMM (DITRON AG-MoE; talk, "MoE dynamic sorting").

Each function states the passage it follows.  Pins (independent checks of these
functions) live in ``tests/test_oracle_*.py``.  Parity unpinned: none of the
functions here -- every one has at least one independent pin.
"""
