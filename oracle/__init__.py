"""CPU oracle for the MC2 compute core: plain, slow, float64/int64.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The HIP library never
calls it, and it never calls the HIP library: the two share no code. Both take
their inputs from ``workloads.py``, which holds only seeded random draws.

Each function is the plain definition of what the operator computes, written
from the pages (cited per module):

* ``gemm.mm_rs`` / ``gemm.ag_mm`` / ``gemm.chunk_rows`` / ``gemm.chunk_order``
  -- MatmulReduceScatter (basic and quantized) and AllGatherMatmul;
* ``moe.histc`` / ``moe.permute`` / ``moe.gmm`` / ``moe.swiglu`` /
  ``moe.dispatch`` / ``moe.combine`` / ``moe.unpermute`` / ``moe.moe_local`` --
  the expert-parallel dispatch/combine local path;
* ``numerics.decode`` / ``numerics.round_to`` -- storage decoding and single
  round-to-nearest-even.

Pins (tests marked ``not gpu``): brute-force loops on tiny shapes, hand-worked
fixtures under ``tests/golden/``, closed forms (power-of-two dequant scales,
SwiGLU limits), invariants (chunks concatenate to the full product, the
simulated reduce-scatter equals one matmul over the concatenated K, counts sum
to T*K, permute then unpermute is the identity), and independent library
routines (``torch.histc``, ``numpy.bincount``, integer matmul, the float32 ->
bf16 and float64 -> float16 casts). Every function here is pinned.
"""
from . import gemm, moe, numerics  # noqa: F401
