"""CPU oracle of the LSA hot path: test infrastructure, never used by the product path."""
from .lsa_oracle import *  # noqa: F401,F403
from .lsa_oracle import (Index, IndexParams, SelectParams, attend, attend_backward, attend_lse,
                         bf16_to_f64, build_index, sparse_attention_backward,
                         bucket_keys, candidates, dense_select, eligible_keys, kmeans, pool,
                         rhe_div, round_bf16, scores, select, sq_dist)
