"""Pins for the oracle attention (CPU only).

The oracle is masked softmax attention over the frame-block mask.  It is
pinned to things other than itself:

* brute force written with plain Python loops and ``math.exp`` on tiny
  inputs (no matmul, no torch softmax) -- catches transposed operands, wrong
  softmax axis, wrong scale;
* the dense N×N form with an explicit token-level mask;
* the library routine ``scaled_dot_product_attention`` in float64 for the
  dense case C ≥ T;
* closed forms: K ≡ 0 gives the mean of V over the attended tokens (with a
  one-hot-by-frame V this reads the mask back as 1/|A(t)| per attended
  frame); V ≡ 1 gives 1; a common offset on every key shifts each row's
  scores by a constant and leaves the output unchanged; an extreme scale
  turns the softmax into a selection of the best-scoring attended key.

Mutation tests plant plausible mistakes in the oracle and check a pin fails.
"""

import math

import pytest
import torch

import oracle
import oracle.attention as oa
import oracle.mask as om
from block_sparse_attention_lvsa_amd.synth import WORKLOADS, make_qkv, make_random

TINY = WORKLOADS["tiny"]


def loops_attention_row(q, k, v, rows, b, h, i, scale):
    """One output row by plain Python loops (float64 via Python floats)."""
    N, d = q.shape[2], q.shape[3]
    T = len(rows)
    P = N // T
    qi = [float(x) for x in q[b, h, i]]
    toks = [j for f in rows[i // P] for j in range(f * P, (f + 1) * P)]
    scores = []
    for j in toks:
        kj = k[b, h, j]
        scores.append(scale * sum(qi[c] * float(kj[c]) for c in range(d)))
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    z = sum(w)
    out = [0.0] * d
    for wj, j in zip(w, toks):
        vj = v[b, h, j]
        for c in range(d):
            out[c] += wj * float(vj[c])
    return [o / z for o in out]


def small_problem(seed=11, B=1, H=2, T=6, P=5, d=8):
    q = make_random((B, H, T * P, d), seed)
    k = make_random((B, H, T * P, d), seed + 1)
    v = make_random((B, H, T * P, d), seed + 2)
    return q, k, v


def _pins_attention():
    """All attention pins on small problems; True when they pass."""
    ok = True
    q, k, v = small_problem()
    rows = om.key_frames(6, 3, 1, 1)
    out = oa.block_attention(q, k, v, rows)
    for (b, h, i) in [(0, 0, 0), (0, 1, 7), (0, 1, 29), (0, 0, 17)]:
        ref = loops_attention_row(q, k, v, rows, b, h, i, 1 / math.sqrt(8))
        ok &= bool(torch.allclose(out[b, h, i], torch.tensor(ref, dtype=torch.float64), atol=1e-12, rtol=0))
    ok &= bool(torch.allclose(out, oa.token_mask_attention(q, k, v, rows), atol=1e-12, rtol=0))
    dense_rows = om.key_frames(6, 6, 2, 0)
    o2 = oa.block_attention(q, k, v, dense_rows)
    ref2 = torch.nn.functional.scaled_dot_product_attention(
        q.double(), k.double(), v.double())
    ok &= bool(torch.allclose(o2, ref2, atol=1e-12, rtol=0))
    return ok


def test_loops_brute_force_and_token_mask():
    assert _pins_attention()


@pytest.mark.parametrize("flags", [om.ROT_MOD_TPER, om.ROT_MOD_T])
def test_tiny_workload_all_steps_vs_token_mask(flags):
    q, k, v = make_qkv(TINY)
    for s in TINY.steps:
        rows = om.key_frames(TINY.T, TINY.C, TINY.W, s, flags)
        a = oa.block_attention(q, k, v, rows)
        b = oa.token_mask_attention(q, k, v, rows)
        assert (a - b).abs().max().item() < 1e-12


def test_tiny_workload_rows_vs_loops():
    q, k, v = make_qkv(TINY)
    rows = om.key_frames(TINY.T, TINY.C, TINY.W, 3)
    out = oa.block_attention(q, k, v, rows)
    for (h, i) in [(0, 0), (1, 200), (1, 511), (0, 447)]:
        ref = loops_attention_row(q, k, v, rows, 0, h, i, 0.125)
        assert torch.allclose(out[0, h, i], torch.tensor(ref, dtype=torch.float64), atol=1e-12, rtol=0)


def test_rows_variant_matches_full():
    q, k, v = make_qkv(TINY)
    rows = om.key_frames(TINY.T, TINY.C, TINY.W, 5)
    full = oa.block_attention(q, k, v, rows)
    toks = [0, 63, 64, 300, 511]
    part = oa.block_attention_rows(q, k, v, rows, 0, 1, toks)
    assert torch.equal(part, full[0, 1, toks]) or (part - full[0, 1, toks]).abs().max() < 1e-14


def test_dense_case_equals_sdpa():
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w)
    rows = om.key_frames(w.T, w.T, 2, 0)  # C = T: dense
    out = oa.block_attention(q, k, v, rows)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double())
    assert (out - ref).abs().max().item() < 1e-12


def test_closed_form_zero_keys_reads_mask():
    T, P, d = 8, 16, 64
    w = WORKLOADS["tiny"]
    q = make_random((1, 1, T * P, d), 5)
    k = torch.zeros(1, 1, T * P, d, dtype=torch.bfloat16)
    v = torch.zeros(1, 1, T * P, d, dtype=torch.bfloat16)
    for j in range(T * P):
        v[0, 0, j, j // P] = 1.0
    for s in range(4):
        rows = om.key_frames(T, w.C, w.W, s)
        out = oa.block_attention(q, k, v, rows)
        for t in range(T):
            expect = torch.zeros(d, dtype=torch.float64)
            for f in rows[t]:
                expect[f] = 1.0 / len(rows[t])
            assert torch.allclose(out[0, 0, t * P:(t + 1) * P], expect.expand(P, d), atol=1e-15, rtol=0)


def test_closed_form_unit_values():
    q, k, _ = small_problem(seed=21)
    v = torch.ones_like(q)
    rows = om.key_frames(6, 3, 1, 2)
    out = oa.block_attention(q, k, v, rows)
    assert (out - 1.0).abs().max().item() < 1e-14


def test_key_offset_invariance():
    q, k, v = small_problem(seed=31)
    u = torch.randn(8, dtype=torch.float64) * 4.0
    rows = om.key_frames(6, 3, 1, 0)
    a = oa.block_attention(q, k, v, rows)
    b = oa.block_attention(q.double(), k.double() + u, v.double(), rows)
    assert (a - b).abs().max().item() < 1e-11


def test_extreme_scale_selects_best_key():
    q, k, v = small_problem(seed=41)
    rows = om.key_frames(6, 3, 1, 1)
    out = oa.block_attention(q, k, v, rows, scale=1e6)
    P = 5
    for i in range(30):
        toks = [j for f in rows[i // P] for j in range(f * P, (f + 1) * P)]
        sc = [(float((q[0, 0, i].double() * k[0, 0, j].double()).sum()), j) for j in toks]
        best = max(sc)[1]
        assert torch.allclose(out[0, 0, i], v[0, 0, best].double(), atol=1e-9)


def test_default_scale():
    assert abs(oracle.default_scale(128) - 0.08838834764831845) < 1e-16
    assert oracle.default_scale(64) == 0.125


# ------------------------------------------------------ mutation tests --


def test_mutation_softmax_wrong_axis(monkeypatch):
    def f(Q, K, V, scale):
        S = (Q @ K.transpose(0, 1)) * scale
        E = torch.exp(S - S.max())
        return (E @ V) / E.sum(dim=0, keepdim=True).sum(dim=1, keepdim=True)
    monkeypatch.setattr(oa, "_softmax_weighted_sum", f)
    assert not _pins_attention()


def test_mutation_wrong_scale(monkeypatch):
    orig = oa._softmax_weighted_sum
    monkeypatch.setattr(oa, "_softmax_weighted_sum", lambda Q, K, V, s: orig(Q, K, V, s * s))
    assert not _pins_attention()


def test_mutation_keys_and_values_swapped(monkeypatch):
    orig = oa._softmax_weighted_sum
    monkeypatch.setattr(oa, "_softmax_weighted_sum", lambda Q, K, V, s: orig(Q, V, K, s))
    assert not _pins_attention()


def test_mutation_wrong_frame_gather(monkeypatch):
    orig = oa._frame_tokens
    monkeypatch.setattr(oa, "_frame_tokens", lambda frames, P: orig([(f + 1) % 6 for f in frames], P))
    assert not _pins_attention()
