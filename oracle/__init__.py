"""CPU oracle of the Mamba-2 selective state update.

TEST INFRASTRUCTURE ONLY. The test suite, the package entry's smoke check and
the benchmark's CPU-baseline leg are the only code allowed to import it; the
GPU package never does, and the two share no code.

  ssu_oracle  plain C (fp32, ctypes front end): the reference the GPU path is
              compared against element by element.
  brute64     an independent float64 NumPy version for tiny shapes, one of the
              pins that hold the C oracle in place.
"""
