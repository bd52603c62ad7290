"""CPU oracle (test infrastructure only; see rlq_oracle.py for what it computes).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg import it.
"""

from .rlq_oracle import *  # noqa: F401,F403
from .rlq_oracle import (  # noqa: F401
    Cache, new_cache, quantize_append, decode, extend, attend, attend_partial, lse_merge,
    rotate, tree_sum_f32, group_stats, assign_codes, pack_codes, unpack_codes,
    encode_tokens, dequant, gather_request, lloyd_max_gaussian, quantizer_mse,
    quantizer_response, coupled_gain, bytes_per_token, bf16_bytes_per_token,
    bf16_bits_to_f64, f32_to_bf16_bits,
)
