"""fp64 CPU oracle for MALA (MassAlloc Attention) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, links or calls anything here, and this package imports nothing from
the product path.

Two independent implementations live here:
  * `mala_oracle.c` (built into `_build/libmala_oracle.so`, wrapped by
    `oracle.core`): the reference used for every parity check, OpenMP over
    independent query blocks / key tiles;
  * `oracle.ref_numpy`: a small numpy statement of the same rule, written
    separately, used only to cross-check the C oracle on tiny inputs.
"""
from .core import (build_oracle, oracle_fwd, oracle_fwd_varlen, oracle_bwd, oracle_bwd_varlen,  # noqa: F401
                   oracle_decode, oracle_threads, KEEP_UNVISITED)
