"""CPU oracle for sample packing and document-causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path: the only common module is ``workloads`` (seeded random inputs).

Contents:
  pack_ref   scalar build_pack / build_unpack / unpack_data, in plain Python lists
  attn_ref   fp64 per-document softmax attention, forward and backward (NumPy)
  dense_ref  fp64 attention on the whole row under a dense block-diagonal causal
             mask built the Megatron way (tiny inputs only)
  mask_stats block sparsity of the document-causal mask
  rope_ref   fp64 rotary position embedding of packed rows (positions from
             the packer's indexes)

Every function is pinned by tests under ``tests/test_oracle_*.py`` to values the
pages print, to closed forms, to library routines on special cases, or to brute
force; see each module's header for the pins.
"""
