"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .sdpa_oracle import (attention_decode, attention_forward, attention_forward_rows,
                          brute_force_attention, default_scale, merge_partials)

__all__ = ["attention_decode", "attention_forward", "attention_forward_rows",
           "brute_force_attention", "default_scale", "merge_partials"]
