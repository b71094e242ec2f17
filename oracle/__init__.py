"""CPU oracle (test infrastructure only): see awq_oracle.py."""
from .awq_oracle import (  # noqa: F401
    PACK, W_BIT, validate, pack_int4, unpack_int4, dequant,
    awq_linear_ref, awq_linear_loops,
    dense_linear_ref, dense_linear_loops,
    validate_gidx, dequant_gidx, awq_linear_gidx_ref, awq_linear_gidx_loops, gidx_order,
)
