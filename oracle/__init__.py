"""Oracle for the gated delta rule (GDN) chunked prefill.

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 CPU implementations of what the
HIP library computes, written from the FlashQLA pages' description of the
operator (API sections of the FlashQLA article) and the gated delta rule they
name.  Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import, call or link anything here.  The HIP path
shares no code with this package and never imports it.

Modules:
  token   -- ctypes front end of gdn_oracle.c (token recurrence fwd + reverse
             mode bwd, OpenMP over (sequence, v-head) units): THE oracle.
  chunked -- separately written NumPy chunked (WY) form, fwd + bwd; a pin.
  brute   -- dense-matrix brute force for T <= 16; a pin.

Pinning status: every function here is pinned by tests/test_oracle_pins.py
(brute force, closed forms, invariants, finite differences); none is
"parity unpinned".
"""
