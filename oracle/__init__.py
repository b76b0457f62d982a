"""CPU oracle for the tree-verification step (test infrastructure).

This package is the independent checker of the HIP library.  Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it;
the library and its Python binding never do.  The arithmetic lives in ``oracle.c``
(plain C, double precision, scalar loops); this module only marshals numpy arrays
into it with ctypes.  It shares no code with the GPU path.

Functions and the passages they follow are documented in ``oracle.c``.  The
draft-tree construction (EAGLE-2 expand, rerank and flatten) is the numpy module
``oracle.tree_build``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

NOT_EVALUATED = -2
NONE = -1
BAD_REQUEST = -3
TIE_TEST = 1
TIE_DRAW = 2


def build() -> str:
    """Compile oracle.c with gcc into liboracle.so (no -ffast-math: IEEE fp64)."""
    cmd = ["gcc", "-O2", "-Wall", "-fPIC", "-shared", "-fopenmp", "-o", _LIB_PATH, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> int:
    """Use n OpenMP threads in the parallel loops; returns the count now in effect."""
    lib().oracle_set_threads(ctypes.c_int(int(n)))
    return int(lib().oracle_max_threads())


def mask(parent, n_nodes):
    """Ancestor / child bitmasks and depths.  parent [B, n_max] int32, n_nodes [B]."""
    parent = _c(parent, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    B, n_max = parent.shape
    anc = np.zeros((B, n_max), np.uint64)
    child = np.zeros((B, n_max), np.uint64)
    depth = np.zeros((B, n_max), np.int32)
    valid = np.zeros(B, np.int32)
    rc = lib().oracle_mask(_p(parent), _p(n_nodes), ctypes.c_int32(B), ctypes.c_int32(n_max),
                           _p(anc), _p(child), _p(depth), _p(valid))
    if rc != 0:
        raise ValueError(f"oracle_mask returned {rc}")
    return anc, child, depth, valid


def _bf16_bits(x):
    """Accept a torch bf16 tensor (as uint16 view) or a uint16 numpy array."""
    return _c(x, np.uint16)


def tree_attention(q, k, v, ctx_len, n_nodes, anc, hq, hkv, scale=None, rows=None,
                   block_table=None, page_size=0, n_pages=0, bf16=False):
    """Tree-masked attention in fp64 for the listed (b, i, h) rows (all rows if None).

    q [B, n_max, hq, d]; k, v [B, S_cap, hkv, d] or paged pool [P, page, hkv, d].
    With bf16=True the activations are uint16 arrays holding bf16 bit patterns.
    Returns [n_rows, d] float64.
    """
    if bf16:
        q, k, v = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v)
        dtype = 1
    else:
        q, k, v = _c(q, np.float32), _c(k, np.float32), _c(v, np.float32)
        dtype = 0
    B, n_max, hq_, d = q.shape
    assert hq_ == hq
    ctx_len = _c(ctx_len, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    anc = _c(anc, np.uint64)
    if rows is None:
        rows = np.array([(b, i, h) for b in range(B) for i in range(n_max) for h in range(hq)], np.int32)
    rows = _c(rows, np.int32).reshape(-1, 3)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if block_table is None:
        kv_capacity = k.shape[1]
        bt = None
    else:
        bt = _c(block_table, np.int32)
        kv_capacity = bt.shape[1]
    out = np.zeros((rows.shape[0], d), np.float64)
    rc = lib().oracle_tree_attention(
        _p(q), _p(k), _p(v), ctypes.c_int32(dtype), _p(bt), ctypes.c_int32(page_size),
        ctypes.c_int32(kv_capacity), ctypes.c_int32(n_pages), _p(ctx_len), _p(n_nodes), _p(anc),
        ctypes.c_int32(B), ctypes.c_int32(n_max), ctypes.c_int32(hq), ctypes.c_int32(hkv), ctypes.c_int32(d),
        ctypes.c_double(scale), _p(rows), ctypes.c_int32(rows.shape[0]), _p(out))
    if rc != 0:
        raise ValueError(f"oracle_tree_attention returned {rc}")
    return out


def softmax(logits, T, want_probs=True):
    """Row softmax at temperature T (fp64).  Returns dict of probs, max, sumexp, argmax, valid."""
    logits = _c(logits, np.float32)
    V = logits.shape[-1]
    flat = logits.reshape(-1, V)
    R = flat.shape[0]
    probs = np.zeros((R, V), np.float64) if (want_probs and T > 0) else None
    mx = np.zeros(R, np.float64)
    se = np.zeros(R, np.float64)
    am = np.zeros(R, np.int32)
    valid = np.zeros(R, np.int32)
    rc = lib().oracle_softmax(_p(flat), ctypes.c_int64(R), ctypes.c_int32(V), ctypes.c_double(T), _p(probs),
                              _p(mx), _p(se), _p(am), _p(valid))
    if rc != 0:
        raise ValueError(f"oracle_softmax returned {rc}")
    return {"probs": probs, "max": mx, "sumexp": se, "argmax": am, "valid": valid}


def acceptance_rate(tgt_logits, dft_logits, T, Td):
    """Per-row acceptance rate alpha = sum_x min(p(x), q(x)) of one drafted token
    drawn from q and verified against p (fp64), with p = softmax(target / T) and
    q = softmax(draft / Td).  Tree-verification notes, "Tree Verification 详解"
    parts A and D.1: a chain token passes with probability alpha, so P(L >= k) is the
    product of the first k levels' alpha when the rows do not depend on the drafted
    tokens.  Rows [..., V] fp32; returns an array of the leading shape."""
    p = softmax(tgt_logits, T)["probs"]
    q = softmax(dft_logits, Td)["probs"]
    shape = np.shape(tgt_logits)[:-1]
    return np.minimum(p, q).sum(axis=-1).reshape(shape)


def reject_sample(tgt_logits, dft_logits, T, Td, tokens, parent, n_nodes, u_accept, u_sample,
                  eps=1e-6, mode="lazy"):
    """Tree rejection sampling.  Logits [B, n_max, V] fp32.  Returns dict of
    accepted_child, term_token, tie_flags (all [B, n_max] int32)."""
    tgt = _c(tgt_logits, np.float32)
    B, n_max, V = tgt.shape
    dft = None if dft_logits is None else _c(dft_logits, np.float32)
    tokens = _c(tokens, np.int32)
    parent = _c(parent, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    ua = None if u_accept is None else _c(u_accept, np.float32)
    us = None if u_sample is None else _c(u_sample, np.float32)
    acc = np.zeros((B, n_max), np.int32)
    term = np.zeros((B, n_max), np.int32)
    ties = np.zeros((B, n_max), np.int32)
    rc = lib().oracle_reject_sample(
        _p(tgt), _p(dft), ctypes.c_double(T), ctypes.c_double(Td), _p(tokens), _p(parent), _p(n_nodes),
        _p(ua), _p(us), ctypes.c_int32(B), ctypes.c_int32(n_max), ctypes.c_int32(V), ctypes.c_double(eps),
        ctypes.c_int32(1 if mode == "all" else 0), _p(acc), _p(term), _p(ties))
    if rc != 0:
        raise ValueError(f"oracle_reject_sample returned {rc}")
    return {"accepted_child": acc, "term_token": term, "tie_flags": ties}


def accept_path(accepted_child, term_token, tokens, n_nodes):
    acc = _c(accepted_child, np.int32)
    term = _c(term_token, np.int32)
    tokens = _c(tokens, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    B, n_max = acc.shape
    pn = np.zeros((B, n_max), np.int32)
    ot = np.zeros((B, n_max), np.int32)
    al = np.zeros(B, np.int32)
    rc = lib().oracle_accept_path(_p(acc), _p(term), _p(tokens), _p(n_nodes), ctypes.c_int32(B),
                                  ctypes.c_int32(n_max), _p(pn), _p(ot), _p(al))
    if rc != 0:
        raise ValueError(f"oracle_accept_path returned {rc}")
    return {"path_nodes": pn, "out_tokens": ot, "accept_len": al}


def kv_commit(k, v, ctx_len, n_nodes, path_nodes, accept_len, block_table=None, page_size=0, n_pages=0):
    """Returns (k, v, new_len, freed, block_table) after the commit; the inputs are not
    modified.  k, v: numpy arrays (float32, or uint16 bf16 bit patterns), one layer's
    cache ([B, cap, hkv, d] or a paged pool [P, page, hkv, d]) or every layer's stacked
    on a leading axis."""
    k = np.array(k, copy=True, order="C")
    v = np.array(v, copy=True, order="C")
    assert k.dtype == v.dtype and k.dtype in (np.float32, np.uint16)
    elem = k.dtype.itemsize
    ctx_len = _c(ctx_len, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    path_nodes = _c(path_nodes, np.int32)
    accept_len = _c(accept_len, np.int32)
    B, n_max = path_nodes.shape
    hkv, d = k.shape[-2], k.shape[-1]
    assert k.ndim in (4, 5) and k.shape == v.shape
    n_layers, stride = (k.shape[0], k[0].size) if k.ndim == 5 else (1, 0)
    bt = None if block_table is None else np.array(block_table, np.int32, copy=True, order="C")
    cap = k.shape[-3] if bt is None else bt.shape[1]
    new_len = np.zeros(B, np.int32)
    freed = np.zeros((B, 64), np.int32)
    rc = lib().oracle_kv_commit(_p(k), _p(v), ctypes.c_int32(elem), ctypes.c_int32(n_layers), ctypes.c_int64(stride),
                                _p(bt), ctypes.c_int32(page_size),
                                ctypes.c_int32(cap), ctypes.c_int32(n_pages), _p(ctx_len), _p(n_nodes),
                                _p(path_nodes), _p(accept_len), ctypes.c_int32(B), ctypes.c_int32(n_max),
                                ctypes.c_int32(hkv), ctypes.c_int32(d), _p(new_len), _p(freed))
    if rc not in (0, -2):
        raise ValueError(f"oracle_kv_commit returned {rc}")
    return k, v, new_len, freed, bt


def verify_step(inp, mode="lazy"):
    """The whole step on one input set (a dict as produced by the synthetic generators):
    mask, tree attention (all rows), target and draft softmax statistics, rejection
    sampling and the accepted path."""
    anc, child, depth, valid = mask(inp["parent"], inp["n_nodes"])
    out = {"anc": anc, "child": child, "depth": depth, "valid": valid}
    if inp.get("q") is not None:
        out["attn"] = tree_attention(
            inp["q"], inp["k"], inp["v"], inp["ctx_len"], inp["n_nodes"], anc, inp["hq"], inp["hkv"],
            block_table=inp.get("block_table"), page_size=inp.get("page_size", 0),
            n_pages=inp.get("n_pages", 0), bf16=inp.get("bf16", False))
    T, Td = inp["T"], inp["Td"]
    out["tgt_stats"] = softmax(inp["tgt_logits"], T, want_probs=False)
    if T > 0:
        out["dft_stats"] = softmax(inp["dft_logits"], Td, want_probs=False)
    rs = reject_sample(inp["tgt_logits"], inp["dft_logits"] if T > 0 else None, T, Td, inp["tokens"],
                       inp["parent"], inp["n_nodes"], inp["u_accept"] if T > 0 else None,
                       inp["u_sample"] if T > 0 else None, mode=mode)
    out.update(rs)
    out.update(accept_path(rs["accepted_child"], rs["term_token"], inp["tokens"], inp["n_nodes"]))
    return out
