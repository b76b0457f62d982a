"""Host logic of the verify-latency cost table and of the grid workload that feeds it."""
import json

import numpy as np
import pytest

import synth
import support
from tree_verification_masked_amd.cost_table import CostTable

B_AX, C_AX, N_AX = (1, 2, 4, 8), (1024, 4096, 16384), (16, 32, 64)


def _multilinear(b, c, n):
    # multilinear in (b, c, n): piecewise-multilinear interpolation must reproduce it
    # everywhere, including the linear extension outside the grid
    return 20.0 + 3.0 * b + 0.002 * c + 0.5 * n + 1e-4 * b * c + 0.01 * b * n + 1e-5 * c * n + 1e-6 * b * c * n


def _rows(f=_multilinear):
    return [{"batch": b, "ctx": c, "n_nodes": n, "step_us": f(b, c, n)} for b in B_AX for c in C_AX for n in N_AX]


def test_exact_on_grid_and_multilinear_between():
    t = CostTable.from_rows(_rows()[::-1])  # row order must not matter
    for r in _rows():
        assert t.latency_us(r["batch"], r["ctx"], r["n_nodes"]) == pytest.approx(r["step_us"], rel=1e-12)
    rng = np.random.default_rng(0)
    for _ in range(200):
        b, c, n = rng.uniform(0.5, 12), rng.uniform(256, 32768), rng.uniform(4, 100)
        assert t.latency_us(b, c, n) == pytest.approx(_multilinear(b, c, n), rel=1e-9)


def test_marginal_and_stopping_rule():
    t = CostTable.from_rows(_rows())
    b, c, n = 3, 6000, 20
    slope = 0.5 + 0.01 * b + 1e-5 * c + 1e-6 * b * c  # d latency / d n
    assert t.marginal_us(b, c, n, 4) == pytest.approx(slope, rel=1e-9)
    cost = 4 * slope
    assert t.worth_expanding(1.01 * cost * 0.1, b, c, n, 4, threshold=0.1)
    assert not t.worth_expanding(0.99 * cost * 0.1, b, c, n, 4, threshold=0.1)
    with pytest.raises(ValueError):
        t.marginal_us(b, c, n, 0)


def test_piecewise_not_global_fit():
    # a kink at the middle context: interpolation follows each segment separately
    f = lambda b, c, n: 10.0 + (c if c <= 4096 else 4096 + 5 * (c - 4096)) * 1e-3 * n  # noqa: E731
    t = CostTable.from_rows(_rows(f))
    assert t.latency_us(2, 2048, 32) == pytest.approx(f(2, 2048, 32))
    assert t.latency_us(2, 8192, 32) == pytest.approx(f(2, 8192, 32))


def test_bad_tables(tmp_path):
    rows = _rows()
    with pytest.raises(ValueError):
        CostTable.from_rows(rows[1:])
    with pytest.raises(ValueError):
        CostTable.from_rows(rows + rows[:1])
    p = tmp_path / "t.json"
    p.write_text(json.dumps({"meta": {"what": "x"}, "rows": rows}))
    t = CostTable.load(p)
    assert t.meta["what"] == "x" and t.lat.shape == (4, 3, 3)


def test_single_point_axes():
    t = CostTable([1], [4096], [16, 64], [[[10.0, 40.0]]])
    assert t.latency_us(8, 100000, 32) == pytest.approx(20.0)  # flat along one-point axes


def test_grid_workload_prefixes_are_trees():
    inp = support.make_config(6, seed=3, with_kv=True, grid=(2, 96, 24), vocab_override=64)
    assert inp["block_table"] is None and inp["kv_capacity"] == 96 + 24
    assert np.all(inp["ctx_len"] == 96) and np.all(inp["n_nodes"] == 24)
    for n in (1, 2, 7, 24):
        pt = synth.grid_point(inp, 1, 40, n)
        par = pt["parent"]
        assert par.shape == (1, n) and par[0, 0] == -1 and np.all(par[0, 1:] < np.arange(1, n))
        assert pt["q"].shape[:2] == (1, n) and pt["k"].shape[0] == 1
        assert pt["tgt_logits"].shape == (1, n, 64) and pt["ctx_len"].tolist() == [40]


def test_committed_table_loads():
    import os

    path = os.path.join(os.path.dirname(__file__), "..", "profiles", "verify_cost_table_llama8b_shape.json")
    t = CostTable.load(path)
    assert t.lat.shape == (4, 3, 3) and np.all(t.lat > 0)
    a = CostTable.load(path, key="attention_us")
    # attention grows with the context at every batch size and tree size
    assert np.all(np.diff(a.lat, axis=1) > 0)
