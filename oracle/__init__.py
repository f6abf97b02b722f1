"""fp64 CPU oracle (test infrastructure only; never imported by the library)."""
from .mla_verify_oracle import (  # noqa: F401
    algorithmic_bytes,
    algorithmic_flops,
    ancestors_inclusive,
    attend_rows,
    check_tree,
    lse_merge,
    mla_verify,
    mla_verify_batched,
    to_f64,
    visible_key_count,
)
