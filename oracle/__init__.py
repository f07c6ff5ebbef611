"""CPU oracle for the Infini-attention layer forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The GPU library and its Python binding never do.

* ``infini_oracle`` -- the equations in numpy float64 (the oracle proper).
* ``brute``         -- the same quantities by pure-Python scalar loops, for tiny inputs;
                       a second, independent writing used to pin the oracle.
"""
