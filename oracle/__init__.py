"""fp64 CPU oracle for causal FoX attention (test infrastructure only).

Importable by the test suite, the smoke check and the benchmark's CPU-baseline
leg; never by the product path.  It shares no code with the HIP library.
"""

from .fox_oracle import attn_bwd, attn_decode, attn_decode_paged, attn_decode_ragged, attn_fwd, fwd_bwd_head, fwd_bwd_tail, attn_fwd_rows, fwd_head_rows, logf_cumsum  # noqa: F401
from .brute import brute_decode_head, brute_fwd_head  # noqa: F401
