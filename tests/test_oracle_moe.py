"""Pins of the mixture-of-experts oracle and of the rounding / activation
helpers it uses (CPU only).

PATHWAYS page, section 6.3: sub-examples are routed to the experts holding
different weights, which needs data-dependent exchanges. The readings pinned
here: top-2 with ties to the lower id, softmax over the two kept logits,
bf16 storage of activations, exact-erf GELU, gate-weighted combine.
"""
import math

import numpy as np
import pytest
import torch

import pw_inputs
from oracle import invariants as inv
from oracle import moe
from oracle import numerics as nm


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(11)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.001953125, 1.005859375,
                                  -1.001953125, 3.0e38, 1e-40, -1e-40], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    assert np.array_equal(nm.to_bf16(a).view(np.uint32), ref.view(np.uint32))


def test_gelu_values_and_identity():
    # GELU(1) = Phi(1) = 0.8413447460685429 (standard normal table), GELU(0) = 0
    assert math.isclose(float(nm.gelu(1.0)), 0.8413447460685429, rel_tol=1e-15)
    assert float(nm.gelu(0.0)) == 0.0
    z = np.linspace(-6, 6, 1001)
    assert np.allclose(nm.gelu(z) - nm.gelu(-z), z, rtol=0, atol=1e-14)   # z Phi(z) + z Phi(-z) = z
    for v in (-3.3, -0.7, 0.2, 2.5):
        assert math.isclose(float(nm.gelu(v)), 0.5 * v * (1 + math.erf(v / math.sqrt(2))), rel_tol=1e-14)


def test_gelu_negative_tail_relative_accuracy():
    """GELU(-a) = -a Phi(-a). For large a the asymptotic series of the normal
    tail, Phi(-a) = phi(a) / a (1 - 1/a^2 + 3/a^4 - 15/a^6 + 105/a^8 - ...),
    fixes it to ~945 / a^10 relative; arbitrary-precision erfc (mpmath, 50
    digits) fixes it everywhere. The oracle must hold its relative accuracy
    there (the erf form, 1 + erf(z / sqrt 2), cancels to 0 below z ~ -8)."""
    import mpmath
    for a in (8.0, 10.0, 12.0, 14.0):
        phi = math.exp(-a * a / 2) / math.sqrt(2 * math.pi)
        series = phi / a * (1 - 1 / a**2 + 3 / a**4 - 15 / a**6 + 105 / a**8)
        assert math.isclose(float(nm.gelu(-a)), -a * series, rel_tol=1000 / a**10)
    mpmath.mp.dps = 50
    for z in np.concatenate([-np.geomspace(1e-3, 14.0, 400), np.geomspace(1e-3, 14.0, 400)]):
        ref = float(mpmath.mpf(z) * mpmath.erfc(-mpmath.mpf(z) / mpmath.sqrt(2)) / 2)
        assert math.isclose(float(nm.gelu(z)), ref, rel_tol=1e-13), z


def _tiny(tokens=40, d=8, e=6, h=5, seed=5):
    rng = np.random.default_rng(seed)
    x = nm.to_bf16(rng.standard_normal((tokens, d)).astype(np.float32))
    wr = nm.to_bf16((rng.standard_normal((d, e)) * 0.3).astype(np.float32))
    w1 = nm.to_bf16((rng.standard_normal((e, d, h)) * 0.3).astype(np.float32))
    w2 = nm.to_bf16((rng.standard_normal((e, h, d)) * 0.3).astype(np.float32))
    return x, wr, w1, w2


def test_router_against_explicit_dot_products():
    x, wr, _, _ = _tiny()
    lg = moe.router_logits(x, wr)
    for t in range(0, 40, 7):
        for e in range(6):
            ref = np.float32(math.fsum(float(x[t, k]) * float(wr[k, e]) for k in range(8)))
            assert lg[t, e] == ref


def test_top2_against_brute_force_with_ties():
    rng = np.random.default_rng(2)
    lg = rng.integers(-3, 4, size=(500, 6)).astype(np.float32)   # many ties
    experts, kept = moe.top2(lg)
    for t in range(500):
        row = lg[t].tolist()
        first = max(range(6), key=lambda e: (row[e], -e))
        rest = [e for e in range(6) if e != first]
        second = max(rest, key=lambda e: (row[e], -e))
        assert experts[t].tolist() == [first, second]
        assert kept[t].tolist() == [row[first], row[second]]


def test_gates_equal_renormalised_full_softmax():
    """Softmax over the kept pair equals the full softmax renormalised over it."""
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((200, 64)).astype(np.float32) * 3
    experts, kept = moe.top2(lg)
    g = moe.gates(kept)
    full = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    pair = np.take_along_axis(full, experts, axis=1)
    ref = pair / pair.sum(axis=1, keepdims=True)
    assert np.allclose(g, ref, rtol=2e-7, atol=0)
    assert np.all(g[:, 0] >= g[:, 1])


def test_expert_ffn_against_explicit_loops():
    x, _, w1, w2 = _tiny(tokens=3)
    y = moe.expert_ffn(x, w1[2], w2[2])
    for i in range(3):
        hs = []
        for j in range(5):
            a = np.float32(math.fsum(float(x[i, k]) * float(w1[2][k, j]) for k in range(8)))
            g = np.float32(0.5 * float(a) * (1.0 + math.erf(float(a) / math.sqrt(2.0))))
            hs.append(float(nm.to_bf16(np.array([g], np.float32))[0]))
        for c in range(8):
            o = np.float32(math.fsum(hs[j] * float(w2[2][j, c]) for j in range(5)))
            assert y[i, c] == nm.to_bf16(np.array([o], np.float32))[0]


def test_moe_step_dispatch_and_combine():
    x, wr, w1, w2 = _tiny()
    r = moe.moe_step(x, wr, w1, w2, num_src=4)
    # the dispatch is an exchange of the 2T tuples by expert
    inv.check_exchange(r.dest, 6, r.src_index, r.offsets, r.counts)
    assert np.array_equal(r.dest, r.experts.reshape(-1))
    # explicit per-token combine
    for t in range(40):
        ys = []
        for j in range(2):
            slot = int(np.flatnonzero(r.src_index == 2 * t + j)[0])
            ys.append(r.y[slot].astype(np.float64))
            assert np.array_equal(r.y[slot], moe.expert_ffn(x[t:t + 1], w1[r.experts[t, j]], w2[r.experts[t, j]])[0])
        ref = nm.to_bf16(nm.to_f32(float(r.gates[t, 0]) * ys[0] + float(r.gates[t, 1]) * ys[1]))
        assert np.array_equal(r.out[t], ref)
    # the per-token path gives the same answer
    e2, g2, o2 = moe.moe_tokens(x, wr, w1, w2, [0, 9, 39])
    assert np.array_equal(o2, r.out[[0, 9, 39]]) and np.array_equal(e2, r.experts[[0, 9, 39]])


def test_identical_experts_combine_to_the_expert_output():
    """With every expert holding the same weights the gates sum to one, so the
    combined output is that FFN's output up to one bf16 rounding."""
    x, wr, w1, w2 = _tiny()
    w1s = np.repeat(w1[:1], 6, axis=0)
    w2s = np.repeat(w2[:1], 6, axis=0)
    r = moe.moe_step(x, wr, w1s, w2s)
    y = moe.expert_ffn(x, w1[0], w2[0])
    ulp = np.abs(y) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(r.out - y) <= ulp)


def test_planted_swap_of_gates_is_caught(monkeypatch):
    x, wr, w1, w2 = _tiny()
    good = moe.moe_step(x, wr, w1, w2)
    monkeypatch.setattr(moe, "gates", lambda kept: nm.to_f32(np.exp(kept[:, ::-1] - kept.max(1, keepdims=True))
                                                              / np.exp(kept - kept.max(1, keepdims=True)).sum(1, keepdims=True)))
    bad = moe.moe_step(x, wr, w1, w2)
    assert not np.array_equal(good.out, bad.out)


def test_capacity_drops_by_hand():
    """Four tokens, two experts, capacity 2 (logits chosen so the routing is
    [[0, 1], [0, 1], [1, 0], [0, 1]]): tuples g = 2t + slot go to experts
    0 1 | 0 1 | 1 0 | 0 1. Expert 0 receives g = 0, 2, 5, 6 and keeps 0, 2;
    expert 1 receives g = 1, 3, 4, 7 and keeps 1, 3. Tokens 2 and 3 lose
    both tuples and combine to zero; tokens 0 and 1 are as without a limit."""
    x, wr, w1, w2 = _tiny(tokens=4, e=2)
    logits = np.array([[2.0, 1.0], [3.0, -1.0], [0.0, 0.5], [1.0, 0.25]], np.float32)
    r = moe.moe_step(x, wr, w1, w2, num_src=1, logits=logits, capacity=2)
    assert r.experts.tolist() == [[0, 1], [0, 1], [1, 0], [0, 1]]
    assert r.offsets.tolist() == [0, 2, 4]
    assert r.src_index.tolist() == [0, 2, 1, 3]
    assert r.counts.tolist() == [[4, 4]]                  # routed, before the limit
    assert np.all(r.out[2:] == 0)
    free = moe.moe_step(x, wr, w1, w2, num_src=1, logits=logits)
    assert np.array_equal(r.out[:2], free.out[:2])
    # capacity 3: expert 0 keeps g = 0, 2, 5 (token 2's slot 1), expert 1
    # keeps g = 1, 3, 4 (token 2's slot 0): token 2 is whole again, token 3
    # has no tuple left
    r3 = moe.moe_step(x, wr, w1, w2, num_src=1, logits=logits, capacity=3)
    assert r3.offsets.tolist() == [0, 3, 6]
    assert r3.src_index.tolist() == [0, 2, 5, 1, 3, 4]
    assert np.array_equal(r3.out[:3], free.out[:3]) and np.all(r3.out[3] == 0)


def test_capacity_one_tuple_dropped_keeps_the_other_term():
    """Three tokens, three experts, capacity 2, routing [[0, 1], [0, 2],
    [0, 1]]: expert 0 receives g = 0, 2, 4 and drops g = 4 (token 2's top-1
    tuple); experts 1 (g = 1, 5) and 2 (g = 3) keep everything. Token 2's
    output is its top-2 term alone, bf16(g_1 * y), not renormalised."""
    x, wr, w1, w2 = _tiny(tokens=3, e=3)
    logits = np.array([[2.0, 1.0, 0.0], [2.0, 0.0, 1.0], [2.0, 1.0, 0.0]], np.float32)
    r = moe.moe_step(x, wr, w1, w2, num_src=1, logits=logits, capacity=2)
    assert r.experts.tolist() == [[0, 1], [0, 2], [0, 1]]
    assert r.offsets.tolist() == [0, 2, 4, 5]
    assert r.src_index.tolist() == [0, 2, 1, 5, 3]
    y1 = moe.expert_ffn(x[2:3], w1[1], w2[1])[0]
    assert np.array_equal(r.out[2], nm.to_bf16(nm.to_f32(float(r.gates[2, 1]) * y1.astype(np.float64))))
    free = moe.moe_step(x, wr, w1, w2, num_src=1, logits=logits)
    assert np.array_equal(r.out[:2], free.out[:2]) and not np.array_equal(r.out[2], free.out[2])


def test_capacity_at_or_above_the_largest_count_changes_nothing():
    x, wr, w1, w2 = _tiny()
    free = moe.moe_step(x, wr, w1, w2, num_src=4)
    top = int(free.counts.sum(axis=0).max())
    for c in (top, top + 5):
        r = moe.moe_step(x, wr, w1, w2, num_src=4, capacity=c)
        assert np.array_equal(r.src_index, free.src_index) and np.array_equal(r.out, free.out)
    r = moe.moe_step(x, wr, w1, w2, num_src=4, capacity=top - 1)
    assert r.offsets[-1] == 80 - int((free.counts.sum(axis=0) > top - 1).sum())


def test_moe_inputs_shapes():
    inp = pw_inputs.moe(tokens=64, d=32, experts=8, hidden=16)
    assert inp.x.dtype == torch.bfloat16 and tuple(inp.w1.shape) == (8, 32, 16) and tuple(inp.w2.shape) == (8, 16, 32)
    assert abs(float(inp.w_router.float().std()) - 0.02) < 0.005
