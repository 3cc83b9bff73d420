"""CPU oracle for the batch-invariant AdaLN final modulation (Qwen-Image ``norm_out``).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP path (``invariant_silu_amd/``) and never reads anything the HIP path wrote.

What it computes is written from the pages, not from any code:

* RL-Kernel pull request 538 ("What" section): the operator
  ``scale, shift = (SiLU(temb) @ W^T + b).chunk(2)`` (3072 -> 6144, scale first)
  and ``out = LayerNorm(x, eps=1e-6, no affine) * (1 + scale) + shift``,
  with forward and backward, an independent CPU FP32 reference whose token
  sums are sequential Neumaier sums, and d_scale / d_shift as FP32 token sums.
* miles_diffusion pull request 108, both versions of its text ("Fused-norm
  rounding points" / "Patches"): under autocast the LayerNorm computes and
  returns fp32, (1 + scale) is rounded once to bf16, the modulation runs in
  fp32, and the single bf16 rounding happens at the consumer's input.
* RL-Kernel pull request 538, review thread (token_sum fix): each 32-token tile
  is summed in ascending order with Neumaier compensation, the tile sums and
  corrections are folded level by level, and one final IEEE add gives the
  result (``token_tree.py``).

Modules:
  fpmath      bf16 rounding, sequential Neumaier sums (NSum), ulp helpers
  adaln       forward / backward in three arithmetic modes:
                "fp32"  the oracle (fp32 ops, NSum reductions)
                "fp64"  the fp64 twin used as arbiter (fp64 between the
                        declared storage roundings)
                "exact" fp64 with no rounding anywhere (finite differences)
  token_tree  the pages' 32-token compensated tree and the plain balanced
              32-way tree it replaced (the "has teeth" control)

Parity status of every function is stated in its docstring; functions without
an independent pin say "parity unpinned".
"""
