"""CPU oracle for sliding-window GQA attention and its compact ring cache.

TEST INFRASTRUCTURE ONLY.  Plain fp64 C (``swa_oracle.c``) plus a byte-exact
numpy ring model (``ring_model.py``).  Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import it;
the GPU library shares no code with it and never calls it.

Pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, a library routine (torch SDPA on CPU), brute force on
tiny inputs and hand-derived worked examples under ``tests/golden/``.
"""
