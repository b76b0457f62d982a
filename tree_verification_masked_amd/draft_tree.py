"""EAGLE-2 draft-tree construction on the GPU: device state plus the three library calls.

``DraftTree`` owns the arrays of the trees under construction (one tree per
request), the expand workspace and a status word, and issues
spec_tree_build_init / spec_tree_expand / spec_tree_rerank on one stream.  The
caller runs its drafter between expand rounds: the draft rows it passes to
``expand`` belong to the current frontier, in ``frontier`` order.  The rerank output
(parent, tokens, n_nodes) is the tree the verification step takes.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


class DraftTree:
    def __init__(self, batch: int, cap: int, max_frontier: int, vocab: int, device="cuda"):
        i32 = dict(dtype=torch.int32, device=device)
        self.batch, self.cap, self.R, self.vocab = batch, cap, max_frontier, vocab
        self.parent = torch.zeros((batch, cap), **i32)
        self.token = torch.zeros((batch, cap), **i32)
        self.path = torch.zeros((batch, cap), dtype=torch.int64, device=device)
        self.value = torch.zeros((batch, cap), dtype=torch.float64, device=device)
        self.conf = torch.zeros((batch, cap), dtype=torch.float64, device=device)
        self.count = torch.zeros(batch, **i32)
        self.frontier = torch.zeros((batch, max_frontier), **i32)
        self.frontier_count = torch.zeros(batch, **i32)
        ws = B.spec_tree_expand_workspace_size(batch, max_frontier, vocab)
        if ws == 0:
            raise ValueError("unsupported draft-tree sizes")
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, **i32)

    def state(self):
        return (self.parent, self.token, self.path, self.value, self.conf, self.count, self.frontier,
                self.frontier_count)

    def init(self, root_tokens, stream=None):
        B.spec_tree_build_init(root_tokens, *self.state(), stream=stream)

    def expand(self, draft_logits, T_d: float, top_k: int, select_k: int | None = None, stream=None,
               policy: str = "layer"):
        """draft_logits [batch, max_frontier, vocab] fp32: row j = the drafter at frontier[b][j].
        policy "layer" (EAGLE-2: the next frontier among this round's children) or
        "best_first" (DDTree: among every unexpanded node)."""
        pol = {"layer": B.EXPAND_LAYER, "best_first": B.EXPAND_BEST_FIRST}[policy]
        B.spec_tree_expand(draft_logits, T_d, top_k, top_k if select_k is None else select_k, *self.state(),
                           self.workspace, status=self.status, stream=stream, policy=pol)

    def rerank(self, n_final: int, out=None, stream=None):
        """Returns (parent, tokens, n_nodes, cand_id) of the flattened trees."""
        if out is None:
            dev = self.parent.device
            out = (torch.empty((self.batch, n_final), dtype=torch.int32, device=dev),
                   torch.empty((self.batch, n_final), dtype=torch.int32, device=dev),
                   torch.empty(self.batch, dtype=torch.int32, device=dev),
                   torch.empty((self.batch, n_final), dtype=torch.int32, device=dev))
        parent, tokens, n_nodes, cand_id = out
        B.spec_tree_rerank(self.parent, self.token, self.path, self.value, self.count, parent, tokens, n_nodes,
                           cand_id, status=self.status, stream=stream)
        return out

    def host_state(self) -> dict:
        torch.cuda.synchronize()
        out = {k: getattr(self, k).cpu().numpy() for k in
               ("parent", "token", "path", "value", "conf", "count", "frontier", "frontier_count", "status")}
        out["path"] = out["path"].view(np.uint64)
        return out
