"""Pins of the oracle's tree attention.

The notes on tree verification (part B) state that a node's attention output equals
an ordinary causal run of prompt + Path(root, node).  These tests build that causal
sequence explicitly and compare with torch's scaled_dot_product_attention in fp64 on
the CPU, a library routine written independently of the oracle."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth


def _path(parent, i):
    p = []
    while i >= 0:
        p.append(i)
        i = parent[i]
    return p[::-1]


def _sdpa_last(qrow, keys, vals, scale):
    """Causal attention over a sequence, read at its last position (sees every key)."""
    L = keys.shape[0]
    qs = torch.zeros((1, 1, L, qrow.shape[0]), dtype=torch.float64)
    qs[0, 0, -1] = torch.from_numpy(qrow)
    out = F.scaled_dot_product_attention(qs, torch.from_numpy(keys)[None, None], torch.from_numpy(vals)[None, None],
                                         is_causal=True, scale=scale)
    return out[0, 0, -1].numpy()


def _random_case(seed, B=2, n_max=12, hq=4, hkv=2, d=16, ctx_hi=40):
    rng = np.random.default_rng(seed)
    parent = np.full((B, n_max), -1, np.int32)
    n_nodes = rng.integers(1, n_max + 1, size=B).astype(np.int32)
    for b in range(B):
        for i in range(1, n_nodes[b]):
            parent[b, i] = rng.integers(0, i)
    ctx = rng.integers(0, ctx_hi, size=B).astype(np.int32)
    s_cap = int(ctx.max() + n_max)
    q = rng.standard_normal((B, n_max, hq, d)).astype(np.float32)
    k = rng.standard_normal((B, s_cap, hkv, d)).astype(np.float32)
    v = rng.standard_normal((B, s_cap, hkv, d)).astype(np.float32)
    return parent, n_nodes, ctx, q, k, v


def test_node_equals_causal_run_of_prompt_plus_path():
    for seed in range(4):
        parent, n_nodes, ctx, q, k, v = _random_case(seed)
        B, n_max, hq, d = q.shape
        hkv = k.shape[2]
        anc, _, _, _ = oracle.mask(parent, n_nodes)
        out = oracle.tree_attention(q, k, v, ctx, n_nodes, anc, hq, hkv).reshape(B, n_max, hq, d)
        scale = 1.0 / np.sqrt(d)
        for b in range(B):
            for i in range(n_nodes[b]):
                pos = list(range(ctx[b])) + [ctx[b] + j for j in _path(parent[b], i)]
                for h in range(hq):
                    g = h // (hq // hkv)  # consecutive query heads share a KV head
                    ref = _sdpa_last(q[b, i, h].astype(np.float64), k[b, pos, g].astype(np.float64),
                                     v[b, pos, g].astype(np.float64), scale)
                    np.testing.assert_allclose(out[b, i, h], ref, rtol=0, atol=1e-12)
            assert np.all(out[b, n_nodes[b]:] == 0)


def test_chain_equals_causal_block():
    rng = np.random.default_rng(7)
    n, ctx, hq, hkv, d = 16, 33, 8, 2, 32
    parent = np.arange(-1, n - 1, dtype=np.int32)[None]
    q = rng.standard_normal((1, n, hq, d)).astype(np.float32)
    k = rng.standard_normal((1, ctx + n, hkv, d)).astype(np.float32)
    v = rng.standard_normal((1, ctx + n, hkv, d)).astype(np.float32)
    anc, _, _, _ = oracle.mask(parent, [n])
    out = oracle.tree_attention(q, k, v, [ctx], [n], anc, hq, hkv).reshape(n, hq, d)
    # one causal run over prompt + chain; queries for prompt positions are dummies
    L = ctx + n
    qs = torch.zeros((1, hq, L, d), dtype=torch.float64)
    qs[0, :, ctx:] = torch.from_numpy(q[0].astype(np.float64)).permute(1, 0, 2)
    ks = torch.from_numpy(k[0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    vs = torch.from_numpy(v[0].astype(np.float64)).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    ref = F.scaled_dot_product_attention(qs, ks, vs, is_causal=True)[0, :, ctx:].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_single_node_is_decode_attention():
    rng = np.random.default_rng(9)
    ctx, hq, hkv, d = 100, 4, 4, 64
    q = rng.standard_normal((1, 1, hq, d)).astype(np.float32)
    k = rng.standard_normal((1, ctx + 1, hkv, d)).astype(np.float32)
    v = rng.standard_normal((1, ctx + 1, hkv, d)).astype(np.float32)
    anc, _, _, _ = oracle.mask(np.array([[-1]], np.int32), [1])
    out = oracle.tree_attention(q, k, v, [ctx], [1], anc, hq, hkv).reshape(hq, d)
    for h in range(hq):
        s = k[0, :, h].astype(np.float64) @ q[0, 0, h].astype(np.float64) / np.sqrt(d)
        w = np.exp(s - s.max())
        ref = (w / w.sum()) @ v[0, :, h].astype(np.float64)
        np.testing.assert_allclose(out[h], ref, rtol=0, atol=1e-12)


def test_paged_layout_matches_contiguous():
    parent, n_nodes, ctx, q, k, v = _random_case(11, B=3, ctx_hi=70)
    B, n_max, hq, d = q.shape
    hkv = k.shape[2]
    page = 16
    rng = np.random.default_rng(12)
    need = [-(-(ctx[b] + n_max) // page) for b in range(B)]
    n_pages = sum(need) + 3
    perm = rng.permutation(n_pages)
    bt = np.full((B, max(need)), -1, np.int32)
    pool_k = rng.standard_normal((n_pages, page, hkv, d)).astype(np.float32)
    pool_v = rng.standard_normal((n_pages, page, hkv, d)).astype(np.float32)
    o = 0
    for b in range(B):
        bt[b, :need[b]] = perm[o:o + need[b]]
        o += need[b]
        for t in range(ctx[b] + n_max):
            pool_k[bt[b, t // page], t % page] = k[b, t]
            pool_v[bt[b, t // page], t % page] = v[b, t]
    anc, _, _, _ = oracle.mask(parent, n_nodes)
    ref = oracle.tree_attention(q, k, v, ctx, n_nodes, anc, hq, hkv)
    got = oracle.tree_attention(q, pool_k, pool_v, ctx, n_nodes, anc, hq, hkv, block_table=bt, page_size=page,
                                n_pages=n_pages)
    np.testing.assert_array_equal(got, ref)


def test_bf16_inputs_are_decoded_exactly():
    parent, n_nodes, ctx, q, k, v = _random_case(13)
    B, n_max, hq, d = q.shape
    hkv = k.shape[2]
    qb, kb, vb = synth.to_bf16_bits(q), synth.to_bf16_bits(k), synth.to_bf16_bits(v)
    anc, _, _, _ = oracle.mask(parent, n_nodes)
    got = oracle.tree_attention(qb, kb, vb, ctx, n_nodes, anc, hq, hkv, bf16=True)
    ref = oracle.tree_attention(synth.bf16_bits_to_f32(qb), synth.bf16_bits_to_f32(kb), synth.bf16_bits_to_f32(vb),
                                ctx, n_nodes, anc, hq, hkv)
    np.testing.assert_array_equal(got, ref)
    # the bit decoding agrees with torch's own bf16
    t = torch.from_numpy(q).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(qb), t)
