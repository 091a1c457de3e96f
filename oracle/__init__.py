"""CPU oracle for the NF4 input-gradient GEMM -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (the HIP library and its Python
binding) never does.
"""

from oracle.nf4_oracle import (  # noqa: F401
    NF4_BLOCK,
    NF4_LEVELS,
    codebook_from_quantiles,
    dequant,
    dequant_columns,
    forward,
    grad_a,
    grad_a_bruteforce,
    grad_a_fp16_operands,
    grad_a_fp16_operands_from_weights,
    grad_a_from_weights,
    num_k_blocks,
    pack,
    pack_codes,
    unpack_codes,
)
