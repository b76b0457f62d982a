"""Test support: input sets whose EAGLE-2 trees (workloads 2 and 5) come from the CPU
oracle's tree builder, the reference the GPU builder is tested against."""
import functools

import synth
from oracle import tree_build as tb


def oracle_tree_builder(row_of, root_token, T_d, top_k, depth, n_final):
    """EAGLE-2 expand rounds, rerank and breadth-first flatten on the CPU (fp64)."""
    t, parent, tokens, ids = tb.build_tree(row_of, root_token, T_d, top_k, depth, n_final)
    return parent, tokens, [tb.path_tokens(t, int(i)) for i in ids]


make_config = functools.partial(synth.make_config, tree_builder=oracle_tree_builder)
