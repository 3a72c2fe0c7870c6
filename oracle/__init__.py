"""fp64 CPU oracle of the KDA recurrent-state update.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import anything in this package; the HIP library and
its Python binding never do.

  kda_oracle.c / .h   plain C, token-by-token, OpenMP over (sequence, head)
  kda_oracle.py       ctypes loader for the C oracle
  kda_oracle_np.py    independent NumPy twin and the chunked (WY/UT) form
  kda_metadata.py     plain loops: the per-step batch metadata (token offsets,
                      slot table, chunk offsets, counts)
  build.py            compiles libkda_oracle.so with gcc
"""
