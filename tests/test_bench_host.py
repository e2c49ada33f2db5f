"""Host-side logic of bench.py: the CPU-baseline leg and the parity record it feeds.

No GPU: the "GPU rows" here are the oracle's own outputs, with planted differences.
"""
import numpy as np

import bench
from oracle import msa_oracle as O
from synth.msa_inputs import WORKLOADS, make_inputs


def _rows_from(outs, n):
    """GPU-row arrays in bench's layout (sample order) built from the oracle's chunks."""
    pos = np.concatenate([p for p, _ in outs])
    bi = np.concatenate([r[0] for _, r in outs], axis=2)
    o = np.concatenate([r[1] for _, r in outs], axis=1)
    lse = np.concatenate([r[2] for _, r in outs], axis=2)
    order = bench.sample_order(n)
    where = {int(p): i for i, p in enumerate(pos)}
    take = np.array([where[int(p)] for p in order[:len(pos)]])
    return {"positions": order[:len(pos)], "block_idx": bi[:, :, take].copy(), "o": o[:, take].copy(),
            "lse": lse[:, :, take].copy()}


def test_cpu_baseline_and_parity_record():
    w = WORKLOADS["tiny_n1k"]
    x = make_inputs(w)
    rep, outs = bench.cpu_baseline(w, x, budget_s=60.0, max_positions=200)
    assert rep["kind"] == "oracle" and rep["unit"] == "tokens/s" and rep["value"] > 0
    assert rep["cores"] >= 1 and rep["host_cpus_affinity"] >= 1 and "cpu_model" in rep
    done = sum(len(p) for p, _ in outs)
    assert done == 200
    # the sampled positions are the first `done` of the fixed permutation
    got = np.sort(np.concatenate([p for p, _ in outs]))
    np.testing.assert_array_equal(got, np.sort(bench.sample_order(w.seqlen)[:done]))

    rows = _rows_from(outs, w.seqlen)
    par = bench.parity_report(w, outs, rows)
    assert (par["positions"], par["index_mismatch"], par["near_ties"], par["not_near_ties"]) == (200, 0, 0, 0)
    assert par["max_abs_O"] == 0.0 and par["max_abs_LSE"] == 0.0

    # plant: one index row with a far block, one O element off by 0.01 and one LSE off by
    # 1e-4 at other positions (O and LSE are compared where the selections agree)
    late = [i for i, p in enumerate(rows["positions"]) if p // 128 >= 5][0]
    other = [i for i in range(len(rows["positions"])) if i != late]
    rows["o"][0, other[0], 1, 5] += 0.01
    rows["lse"][0, 2, other[1]] += 1e-4
    p_late = int(rows["positions"][late])
    sel = rows["block_idx"][0, 0, late].copy()
    pooled = O.index_scores(x["q_idx"], x["k_idx"], positions=[p_late])[0, 0, 0]
    unselected = [c for c in range(p_late // 128) if c not in sel]
    sel[0] = min(unselected, key=lambda c: pooled[c])
    rows["block_idx"][0, 0, late] = np.sort(sel)
    par = bench.parity_report(w, outs, rows)
    assert par["index_mismatch"] == 1 and par["near_ties"] == 0 and par["not_near_ties"] == 1
    assert abs(par["max_abs_O"] - 0.01) < 1e-9
    assert abs(par["max_abs_LSE"] - 1e-4) < 1e-9
