"""Host-side checks of the C-ABI library that need no GPU: it loads, exports every
function the public header declares, and rejects bad arguments before launching."""
import ctypes
import os
import re

import pytest

from tree_verification_masked_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spec_tree.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libspectree.so not built")
    return binding.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 21, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding._SIGNATURES), "binding and header disagree"


def test_version(lib):
    assert "gfx950" in binding.spec_tree_version()


def test_workspace_queries(lib):
    assert binding.spec_tree_softmax_workspace_size(60, 128256) > 60 * 16 * 12
    assert binding.spec_tree_softmax_workspace_size(0, 10) == 0
    a = binding.spec_tree_attention_workspace_size(1, 60, 32, 8, 128, 4156)
    assert a >= 60 * 32 * 130 * 4
    assert binding.spec_tree_attention_workspace_size(1, 60, 30, 8, 128, 4156) == 0  # hq % hkv


P = ctypes.c_void_p(16)  # never dereferenced: every call below fails host validation first


def test_host_errors_mask_and_path(lib):
    assert lib.spec_tree_mask_build(None, P, 1, 7, P, P, P, None, None) == -1
    assert lib.spec_tree_mask_build(P, P, 1, 65, P, P, P, None, None) == -1
    assert lib.spec_tree_mask_build(P, P, 0, 7, P, P, P, None, None) == -1
    assert lib.spec_accept_path(P, P, P, P, 1, 0, P, P, P, None, None) == -1
    assert lib.spec_accept_path(P, None, P, P, 1, 4, P, P, P, None, None) == -1


def test_host_errors_softmax(lib):
    f = lib.spec_tree_softmax
    assert f(P, 4, 100, -1.0, P, P, P, None, None, None, P, 1 << 20, None, None) == -1       # T < 0
    assert f(P, 4, 100, float("nan"), P, P, P, None, None, None, P, 1 << 20, None, None) == -1
    assert f(P, 4, 100, 1.0, P, None, P, None, None, None, P, 1 << 20, None, None) == -1     # T > 0 needs sums
    assert f(P, 4, 100, 1.0, P, P, P, None, None, None, P, 8, None, None) == -5              # workspace
    assert f(P, 4, 100, 1.0, P, P, P, None, None, None, None, 0, None, None) == -5
    g = lib.spec_tree_softmax_pair
    #          tl T    dl Td   R  V    par  nn   nmx tmx tse tam tcm   tcs   dmx dse dcm   dcs   ws wsb      st    s
    ok_rows = [P, 1.0, P, 1.0, 4, 100, None, None, 0, P, P, P, None, None, P, P, None, None, P, 1 << 20, None, None]
    ok_chunks = [P, 1.0, P, 1.0, 4, 100, None, None, 0, None, None, None, P, P, None, None, P, P, P, 1 << 20, None,
                 None]

    def pair(base, **kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return g(*a)

    assert pair(ok_rows, a3=0.0) == -1                      # T_d = 0
    assert pair(ok_rows, a2=None) == -1                     # draft logits
    assert pair(ok_rows, a19=8) == -5                       # workspace
    assert pair(ok_rows, a10=None) == -1                    # row outputs all or none
    assert pair(ok_chunks, a13=None) == -1                  # a chunk pair is both or neither
    assert pair(ok_chunks, a16=None, a17=None) == -1        # chunk pass only: both pairs needed
    assert pair(ok_chunks, a11=P) == -1                     # the argmax needs the row merge
    assert pair(ok_chunks, a19=8) == -5
    # the tree: parent and n_nodes both or neither, chunk partials only, rows = batch x n_max
    assert pair(ok_chunks, a6=P) == -1
    assert pair(ok_chunks, a7=P, a8=4) == -1
    assert pair(ok_rows, a6=P, a7=P, a8=4) == -1            # with row statistics
    assert pair(ok_chunks, a6=P, a7=P, a8=0) == -1          # n_max outside [1, 64]
    assert pair(ok_chunks, a6=P, a7=P, a8=65) == -1
    assert pair(ok_chunks, a6=P, a7=P, a8=3) == -1          # 4 rows are not whole requests of 3 nodes
    assert lib.spec_tree_softmax_chunk() == 4096


def test_host_errors_attention(lib):
    f = lib.spec_tree_attention
    base = dict(q=P, k=P, v=P, dtype=1, bt=None, ps=0, cap=100, npg=0, ctx=P, n=P, par=None, anc=P, B=1, nmax=8,
                hq=8, hkv=2, D=128, maxlen=100, scale=0.1, out=P, ws=P, wsb=1 << 30, st=None, s=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())

    assert call(hq=6, hkv=4) == -1
    assert call(D=96) == -2
    assert call(dtype=7) == -2
    assert call(nmax=65) == -1
    assert call(q=None) == -1
    assert call(scale=0.0) == -1
    assert call(bt=P, ps=0) == -1
    assert call(par=P) == -1            # both the parent links and the ancestor rows
    assert call(anc=None) == -1         # neither
    assert call(par=P, anc=None, wsb=16) == -5  # the parent links alone are accepted
    assert call(wsb=16) == -5


def test_host_errors_reject(lib):
    f = lib.spec_tree_reject_sample
    #       tl T    tmx tam tcm tcs dl Td   dcm dcs tok par nn ua us B  nmax V    acc term pn ot al ws wsb st s
    args = [P, 1.0, None, None, P, P, P, 1.0, P, P, P, P, P, P, P, 1, 8, 100, P, P, None, None, None, None, 0,
            None, None]
    a = list(args)
    a[1] = -0.5
    assert f(*a) == -1
    a = list(args)
    a[7] = 0.0  # T_d must be positive when T > 0
    assert f(*a) == -1
    a = list(args)
    a[1] = 0.0  # greedy needs the row maxima and the argmax
    assert f(*a) == -1
    a[2] = P
    assert f(*a) == -1
    a = list(args)
    a[14] = None  # stochastic needs uniforms
    assert f(*a) == -1
    a = list(args)
    a[16] = 65
    assert f(*a) == -1
    a = list(args)
    a[5] = None  # T > 0 reads the target chunk partials
    assert f(*a) == -1
    a = list(args)
    a[9] = None  # and the draft ones
    assert f(*a) == -1
    a = list(args)
    a[20] = P  # the path outputs come together
    assert f(*a) == -1
    a[21], a[22] = P, P
    assert f(*a) == -5  # all three given: accepted, then the missing workspace
    assert f(*args) == -5  # T > 0 needs the workspace (per-node results)
    a = list(args)
    a[17] = 100000
    assert f(*a) == -5
    a = list(args)
    a[17] = 256 * 4096 + 1  # more than 256 chunks
    assert f(*a) == -2
    assert 0 < binding.spec_tree_reject_sample_workspace_size(1, 60, 4096) < 16384
    assert binding.spec_tree_reject_sample_workspace_size(1, 65, 4096) == 0
    ws = binding.spec_tree_reject_sample_workspace_size(1, 60, 128256)
    assert 60 * 4 * 32 * 8 < ws < 128 * 1024  # each node's level words: two levels x 32 chunks x (P, Q)


def test_host_errors_verify_step(lib):
    """The argument struct's layout agrees with the library's, and the composite step
    refuses bad arguments before launching anything (every case below fails in the
    attention's checks, the first of the three calls)."""
    assert binding.spec_tree_step_args_size() == ctypes.sizeof(binding.SpecTreeStepArgs)
    f = lib.spec_tree_verify_step
    assert f(None, None) == -1
    a = binding.SpecTreeStepArgs(parent=P, tokens=P, n_nodes=P, batch=1, n_max=8, q=P, k=P, v=P, dtype=1,
                                 kv_capacity=4096, ctx_len=P, hq=32, hkv=8, head_dim=128, max_kv_len=4096,
                                 scale=0.088, attn_out=P, attn_workspace=None, attn_workspace_bytes=0,
                                 tgt_logits=P, vocab=1000, temperature=1.0, draft_temperature=1.0)
    assert f(ctypes.addressof(a), None) == -5  # the attention's workspace
    a.q = None
    assert f(ctypes.addressof(a), None) == -1
    a.q = P
    a.head_dim = 96
    assert f(ctypes.addressof(a), None) == -2
    a.head_dim = 128
    a.parent = None  # the step builds the ancestor rows from the parent links
    assert f(ctypes.addressof(a), None) == -1
    # T = 0: the walk runs in the logit pass's launch, so its arguments are checked
    # before anything is launched
    a.parent = P
    a.temperature = 0.0
    a.attn_workspace, a.attn_workspace_bytes = P, 1 << 30  # (the attention's checks would pass)
    assert f(ctypes.addressof(a), None) == -1  # no tgt_max / tgt_argmax / outputs
    a.tgt_max, a.tgt_argmax, a.accepted_child, a.term_token = P, P, P, P
    a.path_nodes = P  # the path outputs come together
    assert f(ctypes.addressof(a), None) == -1
    a.path_nodes = None
    assert f(ctypes.addressof(a), None) == -5  # the logit workspace
    a.softmax_workspace = P
    a.softmax_workspace_bytes = binding.spec_tree_softmax_pair_workspace_size(8, 1000) - 1
    assert f(ctypes.addressof(a), None) == -5
    a.n_max = 65
    assert f(ctypes.addressof(a), None) == -1


def test_host_errors_kv_commit(lib):
    f = lib.spec_tree_kv_commit
    #       k  v  dt nly lstr  bt    ps cap np ctx nn path al B  nmax hkv D    nl fr    st    s
    args = [P, P, 1, 1,  0,    None, 0, 100, 0, P, P, P, P, 1, 8, 8, 128, P, None, None, None]
    for i, bad in ((0, None), (9, None), (17, None)):
        a = list(args)
        a[i] = bad
        assert f(*a) == -1
    a = list(args)
    a[14] = 65  # n_max
    assert f(*a) == -1
    a = list(args)
    a[5], a[6] = P, 0  # block table without a page size
    assert f(*a) == -1
    a = list(args)
    a[3] = 0  # no layers
    assert f(*a) == -1
    a = list(args)
    a[3], a[4] = 2, 100 * 8 * 128 - 1  # layers that would overlap (one layer is 100 x 8 x 128 elements)
    assert f(*a) == -1
    a = list(args)
    a[16] = 96  # head_dim
    assert f(*a) == -2
    a = list(args)
    a[2] = 5  # dtype
    assert f(*a) == -2
    a = list(args)
    a[2], a[15] = 0, 65  # 65 heads x 128 fp32 above the 32 KiB staged per row
    assert f(*a) == -2


def test_host_errors_tree_build(lib):
    f = lib.spec_tree_build_init
    assert f(P, 1, 1025, 4, P, P, P, P, P, P, P, P, None) == -1  # cap above 1024
    assert f(P, 1, 64, 17, P, P, P, P, P, P, P, P, None) == -1   # frontier above 16
    assert f(None, 1, 64, 4, P, P, P, P, P, P, P, P, None) == -1
    g = lib.spec_tree_expand
    #       lg V     T    B  R  k  sk pol cap par tok path val conf cnt fr fc ws wsb      st    s
    args = [P, 1000, 1.0, 1, 4, 4, 4, 0,  64, P, P, P, P, P, P, P, P, P, 1 << 30, None, None]
    for i, bad in ((2, 0.0), (2, float("inf")), (5, 17), (5, 0), (6, 5), (1, 3), (8, 2000), (4, 17), (7, 2)):
        a = list(args)
        a[i] = bad
        assert g(*a) == -1, (i, bad)
    a = list(args)
    a[1] = 64 * 4096 + 1  # vocabulary above 64 chunks
    assert g(*a) == -2
    a = list(args)
    a[18] = 16
    assert g(*a) == -5
    assert binding.spec_tree_expand_workspace_size(1, 4, 1000) > 4 * 16 * 8
    assert binding.spec_tree_expand_workspace_size(1, 17, 1000) == 0
    h = lib.spec_tree_rerank
    assert h(P, P, P, P, P, 1, 64, 65, P, P, P, P, None, None) == -1  # n_final above 64
    assert h(P, P, P, P, P, 1, 0, 8, P, P, P, P, None, None) == -1
    assert h(P, P, None, P, P, 1, 64, 8, P, P, P, P, None, None) == -1


def test_record_calls_keeps_only_accepted_calls(lib):
    """A call the library refuses raises and is not recorded; the recording ends with
    its block, also when the block raises; replaying nothing issues nothing."""
    with binding.record_calls() as rec:
        with pytest.raises(binding.SpecTreeError):
            binding._call("spec_tree_mask_build", None, P, 1, 7, P, P, P, None, None)
    assert rec == []
    assert binding._recording is None
    with pytest.raises(RuntimeError):
        with binding.record_calls():
            raise RuntimeError("inside the block")
    assert binding._recording is None
    binding.replay([])
