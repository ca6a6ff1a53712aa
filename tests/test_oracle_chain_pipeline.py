"""Pins of the chain and pipeline oracles (CPU only).

Chain (PATHWAYS page, section 5.1): A = x + 1 then B = x / 2, each result fed
into the next step. Over the reals x_k = 1 + (x_0 - 1) 2^-k; in fp32 the
iteration reaches 1.0 exactly and stays there.

Pipeline (PATHWAYS page, section 5.3 and Table 2; NEST page, Algorithm 1):
GPipe fill and drain over S stages and M microbatches takes M + S - 1 stage
slots.
"""
import math
import os

import numpy as np
import pytest

import pw_inputs
from oracle import chain as ch
from oracle import exchange as ex
from oracle import numerics as nm
from oracle import pipeline as pp


def closed_form(x0, k):
    return 1.0 + (np.asarray(x0, np.float64) - 1.0) * math.ldexp(1.0, -k)


def test_chain_matches_closed_form_within_rounding():
    """Each step rounds once (x + 1 is rounded, halving is exact); the error
    contracts by 2 per step, so it stays below 2^-23 at every step."""
    x0 = pw_inputs.chain_state(64, 128)
    r = ch.chain(x0, 64, record=64)
    for k, xk in enumerate(r.history, start=1):
        err = np.abs(xk.astype(np.float64) - closed_form(x0, k))
        assert err.max() <= 2.0 ** -23, (k, err.max())


def test_chain_fixed_point_and_fires():
    x0 = pw_inputs.chain_state(256, 128)
    r = ch.chain(x0, 10000)
    assert np.all(r.state == np.float32(1.0))
    assert np.all(r.fut_a == 10000) and np.all(r.fut_b == 10000)
    assert np.all(r.fires_a == 10000) and np.all(r.fires_b == 10000)


def test_chain_equals_plain_fp32_iteration():
    """Bit-exact against numpy fp32 arithmetic, step by step (another route)."""
    x0 = pw_inputs.chain_state(128, 128)
    r = ch.chain(x0, 40, record=40)
    x = x0.copy()
    for k in range(40):
        x = (x + np.float32(1)) * np.float32(0.5)
        assert np.array_equal(x.view(np.uint32), r.history[k].view(np.uint32)), k


def test_chain_planted_mistake_is_caught(monkeypatch):
    """A dropped '+1' in the oracle's A breaks the closed-form pin."""
    x0 = pw_inputs.chain_state(8, 16)
    r = ch.chain(x0, 8, a_op=ex.op_affine(1.0, 0.0), record=8)
    err = np.abs(r.history[-1].astype(np.float64) - closed_form(x0, 8)).max()
    assert err > 2.0 ** -23


# --------------------------------------------------------------------------
# Pipeline
# --------------------------------------------------------------------------

@pytest.mark.parametrize("s,m", [(1, 1), (1, 7), (4, 1), (4, 16), (8, 32), (16, 64), (3, 2)])
def test_gpipe_ticks_closed_form(s, m):
    ticks = pp.gpipe_schedule(s, m)
    assert len(ticks) == m + s - 1            # NEST Algorithm 1: (mbs + s - 1) stage slots
    when = {}
    for t, items in enumerate(ticks):
        stages = [st for st, _ in items]
        assert len(stages) == len(set(stages))          # a stage runs one microbatch per slot
        for st, mb in items:
            when[(st, mb)] = t
    assert len(when) == s * m
    for (st, mb), t in when.items():
        if st > 0:
            assert when[(st - 1, mb)] < t                # input produced earlier
        if mb > 0:
            assert when[(st, mb - 1)] < t                # ascending microbatches per stage
        assert t == st + mb                              # lock-step wavefront
    bubble = 1 - (s * m) / (s * (m + s - 1))
    assert math.isclose(bubble, (s - 1) / (m + s - 1))


def _table2_configs():
    path = os.path.join(os.path.dirname(__file__), "golden", "pathways_table2_pipeline_configs.txt")
    rows = []
    for line in open(path):
        line = line.split("#", 1)[0].split()
        if line:
            rows.append((int(line[0]), int(line[1])))
    return rows


def test_gpipe_schedule_on_the_pages_configs():
    """The (S, M) pairs the PATHWAYS page's Table 2 runs: the oracle's GPipe
    schedule takes M + S - 1 slots, every item once, and the bubble is
    (S - 1) / (M + S - 1) of the stage slots (S = 16, M = 64: 15 / 79)."""
    rows = _table2_configs()
    assert rows == [(4, 16), (8, 32), (16, 64)]
    for s, m in rows:
        ticks = pp.gpipe_schedule(s, m)
        assert len(ticks) == m + s - 1
        assert sum(len(t) for t in ticks) == s * m
        idle = s * len(ticks) - s * m
        assert idle * (m + s - 1) == (s - 1) * s * len(ticks)
    assert math.isclose(15 / 79, 0.189873417721519)


def test_stage_against_explicit_loops():
    rng = np.random.default_rng(3)
    h = nm.to_bf16(rng.standard_normal((3, 5)).astype(np.float32))
    w = nm.to_bf16((rng.standard_normal((5, 4)) * 0.5).astype(np.float32))
    out = pp.stage(h, w)
    for i in range(3):
        for j in range(4):
            a = math.fsum(float(h[i, k]) * float(w[k, j]) for k in range(5))
            a32 = float(np.float32(a))
            g = 0.5 * a32 * (1.0 + math.erf(a32 / math.sqrt(2.0)))
            ref = nm.to_bf16(np.array([g], np.float32))[0]
            assert out[i, j] == ref, (i, j)


def test_forward_is_rowwise_and_composes():
    inp = pw_inputs.pipeline(stages=3, microbatches=2, rows=16, d=32)
    x = inp.x.float().numpy()
    w = inp.w.float().numpy()
    full = pp.forward(x[0], w, keep_all=True)
    assert np.array_equal(full[-1], pp.stage(pp.stage(pp.stage(x[0], w[0]), w[1]), w[2]))
    part = pp.forward(x[0][5:9], w)
    assert np.array_equal(part, full[-1][5:9])
