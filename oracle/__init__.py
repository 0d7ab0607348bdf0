"""CPU oracle for the grouped row-scaled NVFP4 amax + cast.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything from this package; the
product path (``nvfp4_block_scaled_group_amd``) never does, and the two share
no code.  ``oracle.py`` wraps the C oracle ``nvfp4_oracle.c``;
``bruteforce.py`` is an independent numpy brute force used to pin it.
"""
