"""Thin ctypes binding over libspectree.so.

Every function keeps the name of the C entry point it wraps, takes torch tensors
that already live on the GPU, checks dtype / shape / contiguity, and passes raw
device pointers plus the current HIP stream.  No arithmetic of the verification
step happens here; PyTorch only provides device memory and streams.  If the
library is missing the first call raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspectree.so")

SPEC_OK = 0
ATTENTION_SCRATCH_BYTES = 16 << 20  # SPEC_TREE_ATTENTION_SCRATCH_BYTES of spec_tree.h
SPEC_F32 = 0
SPEC_BF16 = 1
NODE_NONE = -1
NODE_NOT_EVALUATED = -2
NODE_BAD_REQUEST = -3
ERR_TIMEOUT = -7  # a bounded cross-workgroup wait of the sampler gave up
ERRORS = {
    0: "SPEC_OK", -1: "SPEC_ERR_INVALID_ARG", -2: "SPEC_ERR_UNSUPPORTED", -3: "SPEC_ERR_BAD_TREE",
    -4: "SPEC_ERR_BAD_INPUT", -5: "SPEC_ERR_WORKSPACE", -6: "SPEC_ERR_HIP", -7: "SPEC_ERR_TIMEOUT",
}

_lib = None
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "spec_tree_mask_build": [_VP, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP],
    "spec_tree_attention_workspace_size": [_I32, _I32, _I32, _I32, _I32, _I32],
    "spec_tree_attention": [_VP, _VP, _VP, _I32, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _I32,
                            _I32, _I32, _F32, _VP, _VP, _SZ, _VP, _VP],
    "spec_tree_attention_noalloc": [_VP, _VP, _VP, _I32, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _I32, _I32,
                                    _I32, _I32, _I32, _F32, _VP, _VP, _VP],
    "spec_tree_softmax_chunk": [],
    "spec_tree_softmax_workspace_size": [_I64, _I32],
    "spec_tree_softmax": [_VP, _I64, _I32, _F32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP, _VP],
    "spec_tree_softmax_pair_workspace_size": [_I64, _I32],
    "spec_tree_softmax_pair": [_VP, _F32, _VP, _F32, _I64, _I32, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                               _VP, _VP, _VP, _SZ, _VP, _VP],
    "spec_tree_reject_sample_workspace_size": [_I32, _I32, _I32],
    "spec_tree_reject_sample": [_VP, _F32, _VP, _VP, _VP, _VP, _VP, _F32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32,
                                _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP, _VP],
    "spec_tree_reject_sample_set_wait_limit": [ctypes.c_uint32],
    "spec_accept_path": [_VP, _VP, _VP, _VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP],
    "spec_tree_verify_step": [_VP, _VP],  # (const SpecTreeStepArgs*, stream)
    "spec_tree_step_args_size": [],
    "spec_tree_kv_commit": [_VP, _VP, _I32, _I32, _I64, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _I32, _I32,
                            _I32, _VP, _VP, _VP, _VP],
    "spec_tree_build_init": [_VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "spec_tree_expand_workspace_size": [_I32, _I32, _I32],
    "spec_tree_expand": [_VP, _I32, _F32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                         _VP, _SZ, _VP, _VP],
    "spec_tree_rerank": [_VP, _VP, _VP, _VP, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP],
    "spec_tree_version": [],
}
_RESTYPES = {
    "spec_tree_step_args_size": _SZ,
    "spec_tree_softmax_chunk": _I32,
    "spec_tree_attention_workspace_size": _SZ,
    "spec_tree_softmax_workspace_size": _SZ,
    "spec_tree_softmax_pair_workspace_size": _SZ,
    "spec_tree_reject_sample_workspace_size": _SZ,
    "spec_tree_expand_workspace_size": _SZ,
    "spec_tree_version": ctypes.c_char_p,
    "spec_tree_reject_sample_set_wait_limit": None,
}


class SpecTreeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {code} ({ERRORS.get(code, 'unknown')})")
        self.code = code


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, ctypes.c_int)
        _lib = handle
    return _lib


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _check(t, dtype, shape=None, name="tensor"):
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


_recording = None  # a list while record_calls() is active


def _call(name, *args):
    fn = getattr(lib(), name)
    rc = fn(*args)
    if rc != SPEC_OK:
        raise SpecTreeError(name, rc)
    if _recording is not None:  # the call with its arguments already converted to C types
        _recording.append((name, fn, tuple(None if a is None else t(a) for t, a in zip(fn.argtypes, args))))
    return rc


class record_calls:
    """Context manager: the library calls made inside it (after their checks, with the
    same pointers, sizes and streams) are kept in the list it returns, for replay()."""

    def __enter__(self):
        global _recording
        _recording = []
        return _recording

    def __exit__(self, *exc):
        global _recording
        _recording = None
        return False


def replay(calls):
    """Issue recorded calls again, as recorded: no argument checks or conversions, so
    the host queues them at a fraction of the cost.  The tensors behind the recorded
    pointers must still be alive; the calls' own host errors are still raised."""
    for name, fn, args in calls:
        rc = fn(*args)
        if rc != SPEC_OK:
            raise SpecTreeError(name, rc)


def spec_tree_version() -> str:
    return lib().spec_tree_version().decode()


# ---------------------------------------------------------------- workspace sizes

def spec_tree_attention_workspace_size(batch, n_max, hq, hkv, head_dim, max_kv_len) -> int:
    return int(lib().spec_tree_attention_workspace_size(batch, n_max, hq, hkv, head_dim, max_kv_len))


def spec_tree_softmax_workspace_size(rows, vocab) -> int:
    return int(lib().spec_tree_softmax_workspace_size(rows, vocab))


def spec_tree_softmax_pair_workspace_size(rows, vocab) -> int:
    return int(lib().spec_tree_softmax_pair_workspace_size(rows, vocab))


def spec_tree_softmax_chunk() -> int:
    return int(lib().spec_tree_softmax_chunk())


def spec_tree_reject_sample_workspace_size(batch, n_max, vocab) -> int:
    return int(lib().spec_tree_reject_sample_workspace_size(batch, n_max, vocab))


# ---------------------------------------------------------------- entry points
# Masks travel as int64 tensors holding the uint64 bit patterns.

def spec_tree_mask_build(parent, n_nodes, anc_mask, child_mask, depth, status=None, stream=None):
    B, n_max = parent.shape
    _check(parent, torch.int32, (B, n_max), "parent")
    _check(n_nodes, torch.int32, (B,), "n_nodes")
    _check(anc_mask, torch.int64, (B, n_max), "anc_mask")
    _check(child_mask, torch.int64, (B, n_max), "child_mask")
    _check(depth, torch.int32, (B, n_max), "depth")
    _check(status, torch.int32, (1,), "status")
    _call("spec_tree_mask_build", _ptr(parent), _ptr(n_nodes), B, n_max, _ptr(anc_mask), _ptr(child_mask),
          _ptr(depth), _ptr(status), _stream(stream))


def _attention_args(q, k, v, ctx_len, n_nodes, anc_mask, out, hkv, max_kv_len, block_table, page_size, n_pages,
                    scale, status, parent):
    """The argument list shared by spec_tree_attention, spec_tree_attention_noalloc and
    the attention fields of spec_tree_verify_step (everything before their workspace /
    status arguments), after the checks.  The
    ancestor sets come from exactly one of anc_mask and parent."""
    B, n_max, hq, D = q.shape
    if q.dtype == torch.bfloat16:
        dtype = SPEC_BF16
    elif q.dtype == torch.float32:
        dtype = SPEC_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t, nm in ((k, "k"), (v, "v"), (out, "out")):
        _check(t, q.dtype, None, nm)
    _check(out, q.dtype, (B, n_max, hq, D), "out")
    _check(ctx_len, torch.int32, (B,), "ctx_len")
    _check(n_nodes, torch.int32, (B,), "n_nodes")
    _check(anc_mask, torch.int64, (B, n_max), "anc_mask")
    _check(parent, torch.int32, (B, n_max), "parent")
    if (anc_mask is None) == (parent is None):
        raise ValueError("give exactly one of anc_mask and parent")
    _check(status, torch.int32, (1,), "status")
    if block_table is None:
        if k.shape[0] != B or k.shape[2] != hkv or k.shape[3] != D or k.shape != v.shape:
            raise ValueError("k/v must be [B, kv_capacity, hkv, D]")
        kv_capacity = k.shape[1]
    else:
        _check(block_table, torch.int32, None, "block_table")
        if block_table.shape[0] != B:
            raise ValueError("block_table must be [B, pages_per_request]")
        if k.shape[1] != page_size or k.shape[2] != hkv or k.shape[3] != D or k.shape != v.shape:
            raise ValueError("paged k/v must be [n_pages, page_size, hkv, D]")
        kv_capacity = block_table.shape[1]
        n_pages = k.shape[0] if not n_pages else n_pages
    if scale is None:
        scale = D ** -0.5
    return (_ptr(q), _ptr(k), _ptr(v), dtype, _ptr(block_table), page_size, kv_capacity, n_pages, _ptr(ctx_len),
            _ptr(n_nodes), _ptr(parent), _ptr(anc_mask), B, n_max, hq, hkv, D, max_kv_len, scale, _ptr(out))


def spec_tree_attention(q, k, v, ctx_len, n_nodes, anc_mask, out, workspace, *, hkv, max_kv_len,
                        block_table=None, page_size=0, n_pages=0, scale=None, status=None, stream=None, parent=None):
    """anc_mask: the ancestor rows; or anc_mask=None and parent= the parent links, from
    which the launch builds them itself."""
    args = _attention_args(q, k, v, ctx_len, n_nodes, anc_mask, out, hkv, max_kv_len, block_table, page_size,
                           n_pages, scale, status, parent)
    _call("spec_tree_attention", *args, _ptr(workspace), workspace.numel() * workspace.element_size(),
          _ptr(status), _stream(stream))


def spec_tree_attention_noalloc(q, k, v, ctx_len, n_nodes, anc_mask, out, *, hkv, max_kv_len, block_table=None,
                                page_size=0, n_pages=0, scale=None, status=None, stream=None, parent=None):
    """spec_tree_attention with the split partials in the library's own per-GPU array
    (SPEC_TREE_ATTENTION_SCRATCH_BYTES): no workspace argument, nothing allocated."""
    args = _attention_args(q, k, v, ctx_len, n_nodes, anc_mask, out, hkv, max_kv_len, block_table, page_size,
                           n_pages, scale, status, parent)
    _call("spec_tree_attention_noalloc", *args, _ptr(status), _stream(stream))


def spec_tree_softmax(logits, temperature, row_max, row_sumexp, row_argmax, workspace, probs=None, chunk_max=None,
                      chunk_sum=None, status=None, stream=None):
    V = logits.shape[-1]
    R = logits.numel() // V
    _check(logits, torch.float32, None, "logits")
    _check(row_max, torch.float32, None, "row_max")
    _check(row_sumexp, torch.float32, None, "row_sumexp")
    _check(row_argmax, torch.int32, None, "row_argmax")
    _check(probs, torch.float32, None, "probs")
    _check(chunk_max, torch.float32, None, "chunk_max")
    _check(chunk_sum, torch.float64, None, "chunk_sum")
    _check(status, torch.int32, (1,), "status")
    for t in (row_max, row_sumexp, row_argmax):
        if t is not None and t.numel() != R:
            raise ValueError("row outputs must have one entry per logit row")
    nch = -(-V // spec_tree_softmax_chunk())
    for t in (chunk_max, chunk_sum):
        if t is not None and t.numel() != R * nch:
            raise ValueError("chunk outputs must be [rows, ceil(vocab / chunk)]")
    _call("spec_tree_softmax", _ptr(logits), R, V, float(temperature), _ptr(row_max), _ptr(row_sumexp),
          _ptr(row_argmax), _ptr(probs), _ptr(chunk_max), _ptr(chunk_sum), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _ptr(status), _stream(stream))


def _check_rows(t, dtype, rows, name):
    """A per-row array (None allowed): dtype and one entry per row."""
    _check(t, dtype, None, name)
    if t is not None and t.numel() != rows:
        raise ValueError(f"{name} must have one entry per logit row ({rows}), got {t.numel()}")


def _check_chunks(cmax, csum, rows, vocab, prefix):
    """A chunk-partials pair (both or neither): fp32 maxima and fp64 sums, [rows, nch]."""
    if (cmax is None) != (csum is None):
        raise ValueError(f"{prefix}_chunk_max and {prefix}_chunk_sum come together")
    _check(cmax, torch.float32, None, f"{prefix}_chunk_max")
    _check(csum, torch.float64, None, f"{prefix}_chunk_sum")
    nch = -(-vocab // spec_tree_softmax_chunk())
    for t, nm in ((cmax, "max"), (csum, "sum")):
        if t is not None and t.numel() != rows * nch:
            raise ValueError(f"{prefix}_chunk_{nm} must be [rows, ceil(vocab / chunk)] = [{rows}, {nch}]")


def spec_tree_softmax_pair(tgt_logits, temperature, dft_logits, draft_temperature, tgt_max, tgt_sumexp, tgt_argmax,
                           tgt_chunk_max, tgt_chunk_sum, dft_max, dft_sumexp, workspace, status=None, stream=None,
                           dft_chunk_max=None, dft_chunk_sum=None, parent=None, n_nodes=None):
    """Row statistics (tgt_max, tgt_sumexp, dft_max, dft_sumexp: all or none; tgt_argmax
    optional) and / or chunk partials of both logit arrays in one launch; with no row
    statistics only the chunk pass runs (both chunk pairs required).  Given the tree
    (parent [B, n_max], n_nodes [B]; logits [B, n_max, V]; chunk partials only), the
    draft partials are computed only for the rows of nodes with children."""
    V = tgt_logits.shape[-1]
    R = tgt_logits.numel() // V
    n_max = 0
    if parent is not None or n_nodes is not None:
        if parent is None or n_nodes is None or parent.dim() != 2:
            raise ValueError("the tree needs parent [B, n_max] and n_nodes [B]")
        n_max = parent.shape[1]
        _check(parent, torch.int32, None, "parent")
        _check(n_nodes, torch.int32, (parent.shape[0],), "n_nodes")
        if parent.shape[0] * n_max != R:
            raise ValueError("the tree's node rows must be the logit rows")
    _check(tgt_logits, torch.float32, None, "tgt_logits")
    _check(dft_logits, torch.float32, tuple(tgt_logits.shape), "dft_logits")
    for t, nm in ((tgt_max, "tgt_max"), (tgt_sumexp, "tgt_sumexp"), (dft_max, "dft_max"), (dft_sumexp, "dft_sumexp")):
        _check_rows(t, torch.float32, R, nm)
    _check_rows(tgt_argmax, torch.int32, R, "tgt_argmax")
    _check_chunks(tgt_chunk_max, tgt_chunk_sum, R, V, "tgt")
    _check_chunks(dft_chunk_max, dft_chunk_sum, R, V, "dft")
    _check(status, torch.int32, (1,), "status")
    _call("spec_tree_softmax_pair", _ptr(tgt_logits), float(temperature), _ptr(dft_logits), float(draft_temperature),
          R, V, _ptr(parent), _ptr(n_nodes), n_max, _ptr(tgt_max), _ptr(tgt_sumexp), _ptr(tgt_argmax),
          _ptr(tgt_chunk_max), _ptr(tgt_chunk_sum), _ptr(dft_max), _ptr(dft_sumexp), _ptr(dft_chunk_max),
          _ptr(dft_chunk_sum), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _ptr(status), _stream(stream))


def spec_tree_reject_sample(tgt_logits, temperature, tokens, parent, n_nodes, accepted_child, term_token, *,
                            tgt_max=None, tgt_argmax=None, tgt_chunk_max=None, tgt_chunk_sum=None, dft_logits=None,
                            draft_temperature=1.0, dft_chunk_max=None, dft_chunk_sum=None, u_accept=None,
                            u_sample=None, workspace=None, status=None, stream=None, path_nodes=None,
                            out_tokens=None, accept_len=None):
    """T == 0 reads tgt_max / tgt_argmax; T > 0 the chunk partials of both arrays, the
    draft logits, the uniforms and the workspace."""
    B, n_max, V = tgt_logits.shape
    R = B * n_max
    _check(tgt_logits, torch.float32, (B, n_max, V), "tgt_logits")
    _check(dft_logits, torch.float32, (B, n_max, V), "dft_logits")
    for t, nm in ((tokens, "tokens"), (parent, "parent"), (accepted_child, "accepted_child"),
                  (term_token, "term_token")):
        _check(t, torch.int32, (B, n_max), nm)
    _check(n_nodes, torch.int32, (B,), "n_nodes")
    _check(u_accept, torch.float32, (B, n_max), "u_accept")
    _check(u_sample, torch.float32, (B, n_max), "u_sample")
    _check_rows(tgt_max, torch.float32, R, "tgt_max")
    _check_rows(tgt_argmax, torch.int32, R, "tgt_argmax")
    _check_chunks(tgt_chunk_max, tgt_chunk_sum, R, V, "tgt")
    _check_chunks(dft_chunk_max, dft_chunk_sum, R, V, "dft")
    _check(status, torch.int32, (1,), "status")
    _check(path_nodes, torch.int32, (B, n_max), "path_nodes")
    _check(out_tokens, torch.int32, (B, n_max), "out_tokens")
    _check(accept_len, torch.int32, (B,), "accept_len")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _call("spec_tree_reject_sample", _ptr(tgt_logits), float(temperature), _ptr(tgt_max), _ptr(tgt_argmax),
          _ptr(tgt_chunk_max), _ptr(tgt_chunk_sum), _ptr(dft_logits), float(draft_temperature), _ptr(dft_chunk_max),
          _ptr(dft_chunk_sum), _ptr(tokens), _ptr(parent), _ptr(n_nodes), _ptr(u_accept), _ptr(u_sample), B, n_max, V,
          _ptr(accepted_child), _ptr(term_token), _ptr(path_nodes), _ptr(out_tokens), _ptr(accept_len),
          _ptr(workspace), ws_bytes, _ptr(status), _stream(stream))


def reject_sample_diagnostics(workspace) -> dict:
    """The sampler workspace's cumulative counters (synchronises): exact W(c) levels
    summed over all nodes, and cross-workgroup waits that gave up."""
    w = workspace[:16].view(torch.int32).tolist()
    return {"levels": int(w[0]), "timeouts": int(w[1])}


def spec_tree_reject_sample_set_wait_limit(polls: int) -> None:
    lib().spec_tree_reject_sample_set_wait_limit(int(polls))


class SpecTreeStepArgs(ctypes.Structure):
    """The C struct SpecTreeStepArgs of spec_tree.h, field for field."""
    _fields_ = [
        ("parent", _VP), ("tokens", _VP), ("n_nodes", _VP), ("batch", _I32), ("n_max", _I32),
        ("q", _VP), ("k", _VP), ("v", _VP), ("dtype", _I32), ("block_table", _VP), ("page_size", _I32),
        ("kv_capacity", _I32), ("n_pages", _I32), ("ctx_len", _VP), ("hq", _I32), ("hkv", _I32), ("head_dim", _I32),
        ("max_kv_len", _I32), ("scale", _F32), ("attn_out", _VP), ("attn_workspace", _VP),
        ("attn_workspace_bytes", _SZ), ("tgt_logits", _VP), ("dft_logits", _VP), ("vocab", _I32),
        ("temperature", _F32), ("draft_temperature", _F32), ("tgt_chunk_max", _VP), ("tgt_chunk_sum", _VP),
        ("dft_chunk_max", _VP), ("dft_chunk_sum", _VP), ("tgt_max", _VP), ("tgt_sumexp", _VP), ("tgt_argmax", _VP),
        ("softmax_workspace", _VP), ("softmax_workspace_bytes", _SZ), ("u_accept", _VP), ("u_sample", _VP),
        ("accepted_child", _VP), ("term_token", _VP), ("path_nodes", _VP), ("out_tokens", _VP), ("accept_len", _VP),
        ("sample_workspace", _VP), ("sample_workspace_bytes", _SZ), ("status", _VP),
    ]


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def spec_tree_verify_step(q, k, v, ctx_len, attn_out, attn_workspace, tgt_logits, temperature, tokens, parent,
                          n_nodes, accepted_child, term_token, path_nodes, out_tokens, accept_len, softmax_workspace,
                          *, hkv, max_kv_len, block_table=None, page_size=0, n_pages=0, scale=None, dft_logits=None,
                          draft_temperature=1.0, tgt_chunk_max=None, tgt_chunk_sum=None, dft_chunk_max=None,
                          dft_chunk_sum=None, tgt_max=None, tgt_sumexp=None, tgt_argmax=None, u_accept=None,
                          u_sample=None, sample_workspace=None, status=None, stream=None):
    """The whole step in one call (attention given the parent links, the logit pass
    with the attention's split combine in its launch, the sampler with the accepted
    path).  T > 0: the chunk partials, draft logits, uniforms and sampler workspace;
    T = 0: tgt_max, tgt_sumexp, tgt_argmax.  Returns the argument struct, which must
    stay alive while a recorded copy of the call may be replayed."""
    (qp, kp, vp, dtype, btp, page_size, kv_capacity, n_pages, ctxp, nnp, parp, _, B, n_max, hq, hkv, D, max_kv_len,
     scale, outp) = _attention_args(q, k, v, ctx_len, n_nodes, None, attn_out, hkv, max_kv_len, block_table,
                                    page_size, n_pages, scale, status, parent)
    V = tgt_logits.shape[-1]
    R = B * n_max
    _check(tgt_logits, torch.float32, (B, n_max, V), "tgt_logits")
    _check(dft_logits, torch.float32, (B, n_max, V), "dft_logits")
    for t, nm in ((tokens, "tokens"), (accepted_child, "accepted_child"), (term_token, "term_token"),
                  (path_nodes, "path_nodes"), (out_tokens, "out_tokens")):
        _check(t, torch.int32, (B, n_max), nm)
    _check(accept_len, torch.int32, (B,), "accept_len")
    _check(u_accept, torch.float32, (B, n_max), "u_accept")
    _check(u_sample, torch.float32, (B, n_max), "u_sample")
    _check_rows(tgt_max, torch.float32, R, "tgt_max")
    _check_rows(tgt_sumexp, torch.float32, R, "tgt_sumexp")
    _check_rows(tgt_argmax, torch.int32, R, "tgt_argmax")
    _check_chunks(tgt_chunk_max, tgt_chunk_sum, R, V, "tgt")
    _check_chunks(dft_chunk_max, dft_chunk_sum, R, V, "dft")
    a = SpecTreeStepArgs(
        parent=parp, tokens=_ptr(tokens), n_nodes=nnp, batch=B, n_max=n_max, q=qp, k=kp, v=vp, dtype=dtype,
        block_table=btp, page_size=page_size, kv_capacity=kv_capacity, n_pages=n_pages, ctx_len=ctxp, hq=hq,
        hkv=hkv, head_dim=D, max_kv_len=max_kv_len, scale=scale, attn_out=outp, attn_workspace=_ptr(attn_workspace),
        attn_workspace_bytes=_nbytes(attn_workspace), tgt_logits=_ptr(tgt_logits), dft_logits=_ptr(dft_logits),
        vocab=V, temperature=float(temperature), draft_temperature=float(draft_temperature),
        tgt_chunk_max=_ptr(tgt_chunk_max), tgt_chunk_sum=_ptr(tgt_chunk_sum), dft_chunk_max=_ptr(dft_chunk_max),
        dft_chunk_sum=_ptr(dft_chunk_sum), tgt_max=_ptr(tgt_max), tgt_sumexp=_ptr(tgt_sumexp),
        tgt_argmax=_ptr(tgt_argmax), softmax_workspace=_ptr(softmax_workspace),
        softmax_workspace_bytes=_nbytes(softmax_workspace), u_accept=_ptr(u_accept), u_sample=_ptr(u_sample),
        accepted_child=_ptr(accepted_child), term_token=_ptr(term_token), path_nodes=_ptr(path_nodes),
        out_tokens=_ptr(out_tokens), accept_len=_ptr(accept_len), sample_workspace=_ptr(sample_workspace),
        sample_workspace_bytes=_nbytes(sample_workspace), status=_ptr(status))
    _call("spec_tree_verify_step", ctypes.addressof(a), _stream(stream))
    return a


def spec_tree_step_args_size() -> int:
    """sizeof(SpecTreeStepArgs) as the library was compiled."""
    return int(lib().spec_tree_step_args_size())


def spec_accept_path(accepted_child, term_token, tokens, n_nodes, path_nodes, out_tokens, accept_len, status=None,
                     stream=None):
    B, n_max = accepted_child.shape
    for t, nm in ((accepted_child, "accepted_child"), (term_token, "term_token"), (tokens, "tokens"),
                  (path_nodes, "path_nodes"), (out_tokens, "out_tokens")):
        _check(t, torch.int32, (B, n_max), nm)
    _check(n_nodes, torch.int32, (B,), "n_nodes")
    _check(accept_len, torch.int32, (B,), "accept_len")
    _check(status, torch.int32, (1,), "status")
    _call("spec_accept_path", _ptr(accepted_child), _ptr(term_token), _ptr(tokens), _ptr(n_nodes), B, n_max,
          _ptr(path_nodes), _ptr(out_tokens), _ptr(accept_len), _ptr(status), _stream(stream))


def spec_tree_kv_commit(k, v, ctx_len, n_nodes, path_nodes, accept_len, new_len, freed_pages=None, *,
                        block_table=None, page_size=0, n_pages=0, status=None, stream=None):
    """In place on k, v (and block_table when paged).  k, v: one layer's cache
    ([B, cap, hkv, D] or the paged pool [P, page, hkv, D]), or every layer's, stacked
    on a leading layer axis ([layers, ...]); the layers share the page table."""
    if k.dtype == torch.bfloat16:
        dtype = SPEC_BF16
    elif k.dtype == torch.float32:
        dtype = SPEC_F32
    else:
        raise TypeError(f"k: unsupported dtype {k.dtype}")
    _check(v, k.dtype, tuple(k.shape), "v")
    B, n_max = path_nodes.shape
    hkv, D = k.shape[-2], k.shape[-1]
    if k.dim() == 5:
        n_layers, layer_stride = k.shape[0], k[0].numel()
        per_layer = k.shape[1:]
    elif k.dim() == 4:
        n_layers, layer_stride, per_layer = 1, 0, k.shape
    else:
        raise ValueError("k/v must be [..., hkv, D] with 4 dims, or 5 with a leading layer axis")
    for t, nm in ((path_nodes, "path_nodes"),):
        _check(t, torch.int32, (B, n_max), nm)
    for t, nm in ((ctx_len, "ctx_len"), (n_nodes, "n_nodes"), (accept_len, "accept_len"), (new_len, "new_len")):
        _check(t, torch.int32, (B,), nm)
    _check(freed_pages, torch.int32, (B, 64), "freed_pages")
    _check(status, torch.int32, (1,), "status")
    cap = per_layer[1] if block_table is None else block_table.shape[1]
    if block_table is not None:
        _check(block_table, torch.int32, (B, cap), "block_table")
    _call("spec_tree_kv_commit", _ptr(k), _ptr(v), dtype, int(n_layers), int(layer_stride), _ptr(block_table),
          int(page_size), int(cap), int(n_pages),
          _ptr(ctx_len), _ptr(n_nodes), _ptr(path_nodes), _ptr(accept_len), B, n_max, hkv, D, _ptr(new_len),
          _ptr(freed_pages), _ptr(status), _stream(stream))


# ---------------------------------------------------------------- draft-tree construction
# The state of the trees under construction: int32 parent / token, int64 path keys
# (the uint64 bit patterns), float64 values and confidences, all [B, cap]; int32
# count [B]; int32 frontier [B, max_frontier] and frontier_count [B].

def spec_tree_expand_workspace_size(batch, max_frontier, vocab) -> int:
    return int(lib().spec_tree_expand_workspace_size(batch, max_frontier, vocab))


def _check_state(cand_parent, cand_token, cand_path, cand_value, cand_conf, cand_count, frontier, frontier_count):
    B, cap = cand_parent.shape
    R = frontier.shape[1]
    _check(cand_parent, torch.int32, (B, cap), "cand_parent")
    _check(cand_token, torch.int32, (B, cap), "cand_token")
    _check(cand_path, torch.int64, (B, cap), "cand_path")
    _check(cand_value, torch.float64, (B, cap), "cand_value")
    _check(cand_conf, torch.float64, (B, cap), "cand_conf")
    _check(cand_count, torch.int32, (B,), "cand_count")
    _check(frontier, torch.int32, (B, R), "frontier")
    _check(frontier_count, torch.int32, (B,), "frontier_count")
    return B, cap, R


def spec_tree_build_init(root_token, cand_parent, cand_token, cand_path, cand_value, cand_conf, cand_count, frontier,
                         frontier_count, stream=None):
    B, cap, R = _check_state(cand_parent, cand_token, cand_path, cand_value, cand_conf, cand_count, frontier,
                             frontier_count)
    _check(root_token, torch.int32, (B,), "root_token")
    _call("spec_tree_build_init", _ptr(root_token), B, cap, R, _ptr(cand_parent), _ptr(cand_token), _ptr(cand_path),
          _ptr(cand_value), _ptr(cand_conf), _ptr(cand_count), _ptr(frontier), _ptr(frontier_count), _stream(stream))


EXPAND_LAYER, EXPAND_BEST_FIRST = 0, 1


def spec_tree_expand(draft_logits, T_d, top_k, select_k, cand_parent, cand_token, cand_path, cand_value, cand_conf,
                     cand_count, frontier, frontier_count, workspace, status=None, stream=None, policy=EXPAND_LAYER):
    B, cap, R = _check_state(cand_parent, cand_token, cand_path, cand_value, cand_conf, cand_count, frontier,
                             frontier_count)
    V = draft_logits.shape[-1]
    _check(draft_logits, torch.float32, (B, R, V), "draft_logits")
    _check(workspace, torch.uint8, None, "workspace")
    _check(status, torch.int32, (1,), "status")
    _call("spec_tree_expand", _ptr(draft_logits), V, float(T_d), B, R, int(top_k), int(select_k), int(policy), cap,
          _ptr(cand_parent), _ptr(cand_token), _ptr(cand_path), _ptr(cand_value), _ptr(cand_conf), _ptr(cand_count),
          _ptr(frontier), _ptr(frontier_count), _ptr(workspace), workspace.numel(), _ptr(status), _stream(stream))


def spec_tree_rerank(cand_parent, cand_token, cand_path, cand_value, cand_count, parent, tokens, n_nodes, cand_id,
                     status=None, stream=None):
    B, cap = cand_parent.shape
    n_final = parent.shape[1]
    _check(cand_parent, torch.int32, (B, cap), "cand_parent")
    _check(cand_token, torch.int32, (B, cap), "cand_token")
    _check(cand_path, torch.int64, (B, cap), "cand_path")
    _check(cand_value, torch.float64, (B, cap), "cand_value")
    _check(cand_count, torch.int32, (B,), "cand_count")
    for t, nm in ((parent, "parent"), (tokens, "tokens"), (cand_id, "cand_id")):
        _check(t, torch.int32, (B, n_final), nm)
    _check(n_nodes, torch.int32, (B,), "n_nodes")
    _check(status, torch.int32, (1,), "status")
    _call("spec_tree_rerank", _ptr(cand_parent), _ptr(cand_token), _ptr(cand_path), _ptr(cand_value),
          _ptr(cand_count), B, cap, n_final, _ptr(parent), _ptr(tokens), _ptr(n_nodes), _ptr(cand_id), _ptr(status),
          _stream(stream))
