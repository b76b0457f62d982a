"""One verification step on the GPU: device buffers plus the five library calls.

``VerifyStep`` owns every buffer the step touches (inputs copied to the device
once, outputs, workspaces, the status word) so that ``run()`` allocates nothing
and only issues the library calls, in order, on one stream:

    spec_tree_attention (given the parent links, it builds the ancestor rows
    itself) -> spec_tree_softmax_pair (the chunk partials of the target and draft
    rows in one launch, no row merge; spec_tree_softmax with row statistics on the
    target rows at T = 0) -> spec_tree_reject_sample (which merges each row itself
    and writes the accepted path, the result of spec_accept_path)

With ``one_call()`` the step is the single spec_tree_verify_step call: the same
kernels in three launches, the attention's split combine running inside the logit
pass's launch.  With ``fold_mask=False`` the step runs spec_tree_mask_build first
and the attention reads its ancestor rows.  ``mask()`` and ``path()`` also run the standalone
spec_tree_mask_build and spec_accept_path calls.

The attention output is not an input of the sampling half (the target logits are
given), so the step's dependence graph has two branches after its start: the
attention, and softmax -> rejection sampling (which checks the tree itself).  With
``overlap()`` the first branch runs on a second stream, forked from and joined back
into the caller's stream by events, so the two branches' latencies overlap.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def to_device(inp: dict, device="cuda") -> dict:
    """Copy a synthetic input set (numpy dict of arrays and scalars, as synth.make_config makes it) to the GPU."""
    d = {}
    for key in ("parent", "tokens", "n_nodes", "ctx_len", "block_table"):
        if inp.get(key) is not None:
            d[key] = torch.from_numpy(np.ascontiguousarray(inp[key], np.int32)).to(device)
    for key in ("tgt_logits", "dft_logits", "u_accept", "u_sample"):
        if inp.get(key) is not None:
            d[key] = torch.from_numpy(np.ascontiguousarray(inp[key], np.float32)).to(device)
    if inp.get("q") is not None:
        for key in ("q", "k", "v"):
            a = np.ascontiguousarray(inp[key])
            if inp["bf16"]:
                d[key] = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
            else:
                d[key] = torch.from_numpy(a.astype(np.float32)).to(device)
    for key in ("B", "n_max", "V", "hq", "hkv", "d", "T", "Td", "bf16", "page_size", "n_pages", "kv_capacity"):
        if key in inp:
            d[key] = inp[key]
    d["max_kv_len"] = int(np.max(inp["ctx_len"]) + inp["n_max"])
    return d


class VerifyStep:
    def __init__(self, dev: dict, with_attention: bool = True, fold_mask: bool = True):
        self.d = dev
        self.fold_mask = fold_mask  # the attention builds the ancestor rows from the parent links
        Bn, n_max, V = dev["B"], dev["n_max"], dev["V"]
        cuda = dev["parent"].device
        i32 = dict(dtype=torch.int32, device=cuda)
        f32 = dict(dtype=torch.float32, device=cuda)
        self.T, self.Td = float(dev["T"]), float(dev["Td"])
        self.with_attention = with_attention and dev.get("q") is not None
        self.status = torch.zeros(1, **i32)
        self.anc = torch.zeros((Bn, n_max), dtype=torch.int64, device=cuda)
        self.child = torch.zeros((Bn, n_max), dtype=torch.int64, device=cuda)
        self.depth = torch.zeros((Bn, n_max), **i32)
        if self.with_attention:
            self.attn_out = torch.empty_like(dev["q"])
            ws = B.spec_tree_attention_workspace_size(Bn, n_max, dev["hq"], dev["hkv"], dev["d"], dev["max_kv_len"])
            self.attn_ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=cuda)
        R = Bn * n_max
        self.tmax, self.tsum, self.targ = torch.zeros(R, **f32), torch.zeros(R, **f32), torch.zeros(R, **i32)
        self.dmax, self.dsum = torch.zeros(R, **f32), torch.zeros(R, **f32)
        nch = -(-V // B.spec_tree_softmax_chunk())
        self.tcmax = torch.zeros((R, nch), **f32)
        self.tcsum = torch.zeros((R, nch), dtype=torch.float64, device=cuda)
        self.dcmax = torch.zeros((R, nch), **f32)
        self.dcsum = torch.zeros((R, nch), dtype=torch.float64, device=cuda)
        self.sm_ws = torch.zeros(B.spec_tree_softmax_pair_workspace_size(R, V), dtype=torch.uint8, device=cuda)
        rj = B.spec_tree_reject_sample_workspace_size(Bn, n_max, V)
        self.rj_ws = torch.zeros(max(rj, 256), dtype=torch.uint8, device=cuda)
        self.accepted_child = torch.zeros((Bn, n_max), **i32)
        self.term_token = torch.zeros((Bn, n_max), **i32)
        self.path_nodes = torch.zeros((Bn, n_max), **i32)
        self.out_tokens = torch.zeros((Bn, n_max), **i32)
        self.accept_len = torch.zeros(Bn, **i32)
        self.side = None
        self.composite = False

    def overlap(self, side_stream=None, fork="start"):
        """Run the attention (after the mask build when it is not folded) on
        ``side_stream`` (a new default-priority stream if None), concurrently with the
        caller's stream.  fork "start": beside softmax and sampling; "after_softmax":
        beside the sampling only.  On MI355X at the 60-node / 4k step either is slower
        than one stream (the attention kernel's registers leave no room on its CUs for
        the others' workgroups, so the kernels mostly wait for each other); where the
        attention outlasts the sampling half (long contexts, large batches) the second
        stream is faster.  Returns self."""
        assert fork in ("start", "after_softmax")
        if self.with_attention:
            self.side = side_stream if side_stream is not None else torch.cuda.Stream(self.d["parent"].device)
            self.ev_fork, self.ev_join = torch.cuda.Event(), torch.cuda.Event()
            self.fork = fork
        return self

    def one_call(self):
        """Run the step as one spec_tree_verify_step call (on the caller's stream).
        Needs the attention from the parent links and no second stream.  Returns self."""
        assert self.with_attention and self.fold_mask and self.side is None
        self.composite = True
        return self

    def verify_step(self, stream=None, replica=None):
        """spec_tree_verify_step over this step's buffers; returns its argument struct."""
        d, r = self.d, replica or {}
        tgt = r.get("tgt_logits", d["tgt_logits"])
        common = dict(hkv=d["hkv"], max_kv_len=d["max_kv_len"], block_table=d.get("block_table"),
                      page_size=d.get("page_size", 0), n_pages=d.get("n_pages", 0), status=self.status, stream=stream)
        if self.T > 0:
            extra = dict(dft_logits=r.get("dft_logits", d["dft_logits"]), draft_temperature=self.Td,
                         tgt_chunk_max=self.tcmax, tgt_chunk_sum=self.tcsum, dft_chunk_max=self.dcmax,
                         dft_chunk_sum=self.dcsum, u_accept=d["u_accept"], u_sample=d["u_sample"],
                         sample_workspace=self.rj_ws)
        else:
            extra = dict(tgt_max=self.tmax, tgt_sumexp=self.tsum, tgt_argmax=self.targ)
        return B.spec_tree_verify_step(r.get("q", d["q"]), r.get("k", d["k"]), r.get("v", d["v"]), d["ctx_len"],
                                       self.attn_out, self.attn_ws, tgt, self.T, d["tokens"], d["parent"],
                                       d["n_nodes"], self.accepted_child, self.term_token, self.path_nodes,
                                       self.out_tokens, self.accept_len, self.sm_ws, **common, **extra)

    # the individual stages -------------------------------------------------
    def mask(self, stream=None):
        d = self.d
        B.spec_tree_mask_build(d["parent"], d["n_nodes"], self.anc, self.child, self.depth, self.status, stream)

    def attention(self, stream=None, q=None, k=None, v=None, out=None):
        d = self.d
        B.spec_tree_attention(d["q"] if q is None else q, d["k"] if k is None else k, d["v"] if v is None else v,
                              d["ctx_len"], d["n_nodes"], None if self.fold_mask else self.anc,
                              self.attn_out if out is None else out, self.attn_ws, hkv=d["hkv"],
                              max_kv_len=d["max_kv_len"], block_table=d.get("block_table"),
                              page_size=d.get("page_size", 0), n_pages=d.get("n_pages", 0), status=self.status,
                              stream=stream, parent=d["parent"] if self.fold_mask else None)

    def softmax(self, stream=None, tgt=None, dft=None, rows=False):
        """T > 0: the chunk partials of both logit arrays (one launch), the draft rows
        only of nodes with children (the sampler reads no others); with rows, the row
        statistics of every row as well (a second, merging launch the sampler does not
        need).  T = 0: the target rows' maximum and argmax."""
        d = self.d
        tgt = d["tgt_logits"] if tgt is None else tgt
        if self.T > 0:
            B.spec_tree_softmax_pair(tgt, self.T, d["dft_logits"] if dft is None else dft, self.Td,
                                     self.tmax if rows else None, self.tsum if rows else None,
                                     self.targ if rows else None, self.tcmax, self.tcsum,
                                     self.dmax if rows else None, self.dsum if rows else None, self.sm_ws,
                                     status=self.status, stream=stream, dft_chunk_max=self.dcmax,
                                     dft_chunk_sum=self.dcsum, parent=None if rows else d["parent"],
                                     n_nodes=None if rows else d["n_nodes"])
        else:
            B.spec_tree_softmax(tgt, 0.0, self.tmax, self.tsum, self.targ, self.sm_ws, status=self.status,
                                stream=stream)

    def reject(self, stream=None, tgt=None, dft=None, with_path=True):
        """Rejection sampling; with_path: the same walk also writes the accepted path
        (path_nodes, out_tokens, accept_len), the result spec_accept_path gives."""
        d = self.d
        tgt = d["tgt_logits"] if tgt is None else tgt
        path = dict(path_nodes=self.path_nodes, out_tokens=self.out_tokens, accept_len=self.accept_len) \
            if with_path else {}
        if self.T == 0:
            B.spec_tree_reject_sample(tgt, 0.0, d["tokens"], d["parent"], d["n_nodes"], self.accepted_child,
                                      self.term_token, tgt_max=self.tmax, tgt_argmax=self.targ, status=self.status,
                                      stream=stream, **path)
            return
        B.spec_tree_reject_sample(tgt, self.T, d["tokens"], d["parent"], d["n_nodes"], self.accepted_child,
                                  self.term_token, tgt_chunk_max=self.tcmax, tgt_chunk_sum=self.tcsum,
                                  dft_logits=d["dft_logits"] if dft is None else dft, draft_temperature=self.Td,
                                  dft_chunk_max=self.dcmax, dft_chunk_sum=self.dcsum, u_accept=d["u_accept"],
                                  u_sample=d["u_sample"], workspace=self.rj_ws, status=self.status, stream=stream,
                                  **path)

    def path(self, stream=None):
        d = self.d
        B.spec_accept_path(self.accepted_child, self.term_token, d["tokens"], d["n_nodes"], self.path_nodes,
                           self.out_tokens, self.accept_len, self.status, stream)

    def run(self, stream=None, replica=None):
        """The whole step.  ``replica`` (optional dict) swaps in another copy of the
        large inputs (q/k/v and logits) so that timed loops can rotate buffers."""
        r = replica or {}
        if self.composite:
            self._args = self.verify_step(stream, r)  # (kept alive until the next call)
            return
        if self.side is not None:
            main = torch.cuda.current_stream() if stream is None else stream
            if self.fork == "after_softmax":
                self.softmax(main, r.get("tgt_logits"), r.get("dft_logits"))
            self.ev_fork.record(main)  # the side branch starts after the caller's earlier work
            self.side.wait_event(self.ev_fork)
            if not self.fold_mask:
                self.mask(self.side)
            self.attention(self.side, r.get("q"), r.get("k"), r.get("v"))
            self.ev_join.record(self.side)
            if self.fork == "start":
                self.softmax(main, r.get("tgt_logits"), r.get("dft_logits"))
            self.reject(main, r.get("tgt_logits"), r.get("dft_logits"))
            main.wait_event(self.ev_join)  # the whole step is done when the caller's stream is
            return
        if self.with_attention:
            if not self.fold_mask:
                self.mask(stream)
            self.attention(stream, r.get("q"), r.get("k"), r.get("v"))
        self.softmax(stream, r.get("tgt_logits"), r.get("dft_logits"))
        self.reject(stream, r.get("tgt_logits"), r.get("dft_logits"))  # and the accepted path

    def compile(self, replicas, stream=None):
        """Record the step's library calls for each input replica (running each once),
        so that run_fast(i) issues replica i's step with the recorded arguments and no
        per-call checks.  The recorded streams are the caller's (current) stream and
        this step's side stream.  The recorded calls hold raw device addresses, so the
        replicas (and this step's own buffers) are kept alive with the plans; a buffer
        replaced afterwards needs a new compile().  Returns self."""
        main = torch.cuda.current_stream() if stream is None else stream
        self._main = main
        self._plans = []
        self._replicas = list(replicas)  # keeps every recorded address valid
        self._keep = []
        torch.cuda.synchronize()
        for r in replicas:
            if self.side is not None:
                with B.record_calls() as side_calls:
                    if not self.fold_mask:
                        self.mask(self.side)
                    self.attention(self.side, r.get("q"), r.get("k"), r.get("v"))
                with B.record_calls() as main_calls:  # one softmax call, then the sampler
                    self.softmax(main, r.get("tgt_logits"), r.get("dft_logits"))
                    self.reject(main, r.get("tgt_logits"), r.get("dft_logits"))
                self._plans.append((list(side_calls), list(main_calls)))
            elif self.composite:
                with B.record_calls() as calls:
                    self._keep.append(self.verify_step(main, r))  # the recorded call points at this struct
                self._plans.append(([], list(calls)))
            else:
                with B.record_calls() as calls:
                    self.run(main, r)
                self._plans.append(([], list(calls)))
            torch.cuda.synchronize()
        return self

    def run_fast(self, i):
        """The step of recorded replica i (compile()), forked and joined as run() does."""
        side_calls, main_calls = self._plans[i]
        main = self._main
        if self.side is not None:
            if self.fork == "after_softmax":  # the side branch waits for the logit pass
                B.replay(main_calls[:1])
                main_calls = main_calls[1:]
            self.ev_fork.record(main)
            self.side.wait_event(self.ev_fork)
            B.replay(side_calls)
            self.ev_join.record(self.side)
            B.replay(main_calls)
            main.wait_event(self.ev_join)
        else:
            B.replay(main_calls)

    def results(self) -> dict:
        torch.cuda.synchronize()
        out = {k: getattr(self, k).cpu().numpy() for k in
               ("anc", "child", "depth", "tmax", "tsum", "targ", "dmax", "dsum", "tcmax", "tcsum", "dcmax", "dcsum",
                "accepted_child", "term_token", "path_nodes", "out_tokens", "accept_len", "status")}
        out["anc"] = out["anc"].view(np.uint64)
        out["child"] = out["child"].view(np.uint64)
        if self.with_attention:
            out["attn"] = self.attn_out.float().cpu().numpy()
        return out
