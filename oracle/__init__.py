"""CPU oracle of block-sparse video attention -- test infrastructure only.

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``; the library never imports, links or runs it.  See
``oracle/reference.py`` for the definitions and the pages they follow, and
``oracle/cluster_select.py`` for the intra-block clustering selector,
``oracle/domains.py`` for top-p over competition domains and
``oracle/structured.py`` for the structured (per-head frame context) lists.
"""
from .reference import *  # noqa: F401,F403
from .reference import (Geometry, MaskParams, attention, attention_head, attention_head_gathered,  # noqa: F401
                        block_logits,
                        build_mask, exp_spec, fold_sum, inclusion_probabilities,
                        philox4x64_10, pool_blocks, sample_uniforms, select_sample,
                        select_topk, topk_count, score_scale, forward_scale,
                        log_cluster_table)
from .cluster_select import (block_softmax, cluster_importance, kmeans_block,  # noqa: F401
                             select_blocks, select_sample_weights, water_fill)
