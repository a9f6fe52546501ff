"""CPU oracle for the MSA sparse-prefill path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library never calls it, and it shares no code with the
library.  See ``oracle.msa`` for the functions and what pins each of them.
"""
from .msa import (  # noqa: F401
    PAGE, HEAD_DIM, e4m3_table, decode_e4m3, query_positions, index_scores,
    topk_select, k2q_csr, sparse_attention, round_bf16, bf16_bits_to_float,
    encode_e4m3, quantize_e4m3, insert_index_k, insert_kv,
    Mxfp4Keys, e2m1_table, e8m0_value, decode_mxfp4, encode_e2m1, quantize_mxfp4,
    insert_index_k_mxfp4, Mxfp4KV, mxfp4_staged_table, mxfp4_kv_as_e4m3,
)
