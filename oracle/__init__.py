"""CPU fp64 oracle for the Lightning Attention layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.

Two independent evaluations of the same definition
(o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s + lambda^(t+1) q_t^T S0,
lambda = exp(-slope), Ling & Ring 2.6 Technical Report pages, "Hybrid Linear
Attention" and "Context Parallel for Lightning Attention" sections):

* `fwd`, `decode`, `bwd`, `fwd_chunked` call the plain C recurrent code in
  `la_oracle.c` (fp64, OpenMP over (b, h)); `fwd_varlen` and `bwd_varlen`
  apply them to each sequence of a packed batch;
* `brute` holds the quadratic (masked-matrix) forms in numpy, for tiny sizes;
* `gated_group_rmsnorm` is the output epilogue (per-head RMSNorm, weight,
  sigmoid gate) written out in numpy, and `fwd_gated` composes it with `fwd`.
"""
from .core import (  # noqa: F401
    build,
    fwd,
    fwd_chunked,
    fwd_varlen,
    fwd_gated,
    gated_group_rmsnorm,
    decode,
    bwd,
    bwd_varlen,
    num_threads,
    library_path,
)
from . import brute  # noqa: F401
