"""Plain fp64 CPU oracle of the SparseGPT layer solver.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library.

Sources (cited by page title and section throughout):

* [SGR] "SparseGPT: Massive Language Models Can Be Accurately Pruned in
  One-Shot" -- paper review on devpress.csdn.net.  Sections 6 (the layer-wise
  reconstruction objective), 7 (the Hessian proxy H = X X^T), 8 (Optimal Brain
  Surgeon prune-and-compensate), 11 (the pruning pipeline: column blocks,
  prune a given fraction, update the rest), 14.4 (N:M semi-structured).
* [SFT] "Sparse Fine-tuning for Inference Acceleration of Large Language
  Models" -- review on tqpw.cn.  Section 8.4 (N:M groups: 2:4, 16:32, 16:64,
  16:128 keep N of every M), section 4.2 (compression ratio <-> sparsity).
* [VSG] "Vector-Based SparseGPT" -- press article on voc.com.cn, parts 01-02
  (SparseGPT processes weights in order and compensates the rest; block-wise
  processing passes the error on to later parts).
* [VSG] parts 01-02 also describe vector-level joint compensation: the
  weights chosen within a range are removed together and the kept ones
  adjusted jointly (prune_vector).
* [G24] "LLM 2:4 structured sparsity production guide" -- oh-bug.com, section
  on the 2:4 core mechanism (two zeros in every four consecutive values along
  the reduction axis; the worked example [0.42,-0.18,0.07,0.31]).

Where the pages are silent (damping, the Cholesky route to the inverse factor,
the saliency formula, block size, lazy batching, selection granularity and
timing, ties) the reading adopted is stated at each function.

Pinning: every function is checked in tests/test_oracle_pins.py against
brute force, closed forms, textbook least squares, exhaustive search at n = 8,
the printed 2:4 example and invariances.  One reading has no such pin: the
granularity (whole m x w block) and timing (block start) of multi-weight
unstructured selection -- parity unpinned for that reading; the pages print no
example of it.
"""

from .sparsegpt_oracle import (  # noqa: F401
    Pattern,
    parse_pattern,
    hessian,
    dampen,
    inverse_upper_factor,
    prune,
    prune_free_set,
    reconstruction_error,
    reconstruction_error_from_hessian,
    solve_layer,
    pack_two_four,
    quant_grid,
    quant_code,
    prune_quantized,
    prune_vector,
    unpack_two_four,
    unstructured_k,
)
