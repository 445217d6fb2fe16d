"""CPU oracle (test infrastructure only; never called by the GPU library).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import it.
"""
from .attention import (attention_bruteforce, attention_bwd_fp64,  # noqa: F401
                        attention_dropout_fp64, attention_fp64, attention_rows_fp64,
                        attention_varlen_fp64, dropout_keep_mask, dropout_threshold,
                        head_forward)
