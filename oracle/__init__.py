"""Slow, plain fp64 CPU oracle for learned block-compressed attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything under this directory: only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constant or
table with the HIP library; the only thing both sides consume is the seeded input
generator in ``block_compressed_kv_amd/synth.py``, which holds none of the
method's arithmetic.

Modules
-------
``lbca_oracle``  vectorised fp64 NumPy implementation of every step on the path
                 (visibility, the three pooling forms, decode and prefill
                 attention with the HCA/CSA treatment, the lightning indexer and
                 top-k selection, and the analytic KV accounting).
``brute``        an independently written pure-Python-loop twin for tiny sizes,
                 used only to check ``lbca_oracle``.

Pins: every function is checked in ``tests/test_oracle_*.py`` against values the
pages print (``tests/golden/``), closed forms, invariants and brute force; no
function is without a pin.  The pages print no output values at the workload
sizes, so beyond those pins the fp64 oracle itself is the reference there.
"""
