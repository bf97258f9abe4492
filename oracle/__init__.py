"""CPU oracle for MLA decode (fp64 numpy).  TEST INFRASTRUCTURE: only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it."""
from .mla import *  # noqa: F401,F403
from .mla import (attend_absorbed, attend_causal_chunk, attend_reconstruct, attend_sparse, down_project,  # noqa: F401
                  gqa_equivalent_groups, indexer_scores, sparse_decode, topk_select,
                  mha_cache_elements_per_token, mla_cache_elements_per_token, output_project, query_project,
                  query_project_lowrank, rope, rope_angles, softmax_scale)
