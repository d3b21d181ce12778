"""Pins for the attention oracle (O1). CPU only.

Each test ties the oracle to something other than itself: a library routine
(torch SDPA in fp64), brute force, a second algorithm, closed forms derived by
hand, or values the pages print (tests/golden/)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    qt, kt, vt = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                         is_causal=causal, scale=scale)
    return o[0, 0].numpy()


@pytest.mark.parametrize("n,d", [(1, 8), (37, 16), (128, 64)])
def test_global_equals_sdpa_causal(n, d):
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    scale = 1 / math.sqrt(d)
    mask = A.visibility_mask(W.GLOBAL, 0, 0, None, np.arange(n), n)
    o, _ = A.attend_masked(q, k, v, mask, scale)
    ref = _sdpa(q, k, v, causal=True, scale=scale)
    assert np.max(np.abs(o - ref)) < 1e-12


@pytest.mark.parametrize("n,s,w", [(100, 4, 16), (64, 0, 1), (90, 7, 90), (50, 60, 3)])
def test_local_equals_sdpa_band(n, s, w):
    # the band is built from torch.tril's own diagonal convention: tril(x, k) keeps
    # j <= i + k, so "not tril(-w)" keeps j > i - w; the sink columns are j < s.
    ones = torch.ones(n, n, dtype=torch.bool)
    band = torch.tril(ones) & ~torch.tril(ones, -w)
    sink = torch.tril(ones) & (torch.arange(n)[None, :] < s)
    mask_lib = (band | sink).numpy()
    q, k, v = _rand((n, 32), 4), _rand((n, 32), 5), _rand((n, 32), 6)
    mask = A.visibility_mask(W.LOCAL, s, w, None, np.arange(n), n)
    assert np.array_equal(mask, mask_lib)
    o, _ = A.attend_masked(q, k, v, mask, 0.2)
    ref = _sdpa(q, k, v, mask=mask_lib, scale=0.2)
    assert np.max(np.abs(o - ref)) < 1e-12


CASES = [(W.GLOBAL, 0, 0, None), (W.LOCAL, 3, 5, None), (W.LOCAL, 0, 1, None),
         (W.RETRIEVAL, 0, 0, np.array([2, 3, 11, 20, 29])), (W.RETRIEVAL, 0, 0, np.array([], int))]


@pytest.mark.parametrize("case", CASES)
def test_loops_bruteforce_matches(case):
    kind, s, w, r = case
    n, d = 30, 8
    q, k, v = _rand((n, d), 7), _rand((n, d), 8), _rand((n, d), 9)
    rows = np.arange(n)
    o1, l1 = A.attend_masked(q, k, v, A.visibility_mask(kind, s, w, r, rows, n), 0.35)
    o2, l2 = A.attend_loops(q, k, v, kind, s, w, r, list(rows), 0.35)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    fin = np.isfinite(l2)
    assert np.array_equal(np.isfinite(l1), fin)
    assert np.max(np.abs(l1[fin] - l2[fin]), initial=0) < 1e-12


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("block", [1, 7, 16, 64])
def test_blocked_online_softmax_matches(case, block):
    kind, s, w, r = case
    n, d = 70, 16
    q, k, v = _rand((n, d), 10), _rand((n, d), 11), _rand((n, d), 12)
    mask = A.visibility_mask(kind, s, w, r, np.arange(n), n)
    o1, l1 = A.attend_masked(q, k, v, mask, 0.25)
    o2, l2 = A.attend_blocked(q, k, v, mask, 0.25, block=block)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    assert np.max(np.abs(l1[fin] - l2[fin]), initial=0) < 1e-12


def test_local_sink0_window1_is_identity():
    n = 40
    q, k, v = _rand((n, 8), 13), _rand((n, 8), 14), _rand((n, 8), 15)
    o, lse = A.attend_masked(q, k, v, A.visibility_mask(W.LOCAL, 0, 1, None, np.arange(n), n), 0.5)
    assert np.array_equal(o, v)  # one visible key, weight exactly 1
    assert np.allclose(lse, 0.5 * np.sum(q * k, axis=1), atol=1e-12, rtol=0)


@pytest.mark.parametrize("s,w", [(4, 16), (0, 8), (5, 1), (3, 30)])
def test_local_uniform_mean_closed_form(s, w):
    # q = 0 gives equal weights; with v_j = j the output is the mean visible
    # position. For a row i >= s + w the visible keys are the s sink positions
    # and the w positions i-w+1..i, so by arithmetic series the mean is
    # (s(s-1)/2 + w*i - w(w-1)/2) / (s + w).
    n = 80
    q = np.zeros((n, 4))
    k = _rand((n, 4), 16)
    v = np.repeat(np.arange(n, dtype=np.float64)[:, None], 4, axis=1)
    o, lse = A.attend_masked(q, k, v, A.visibility_mask(W.LOCAL, s, w, None, np.arange(n), n), 1.0)
    for i in range(s + w, n):
        mean = (s * (s - 1) / 2 + w * i - w * (w - 1) / 2) / (s + w)
        assert abs(o[i, 0] - mean) < 1e-9
        assert abs(lse[i] - math.log(s + w)) < 1e-12
    for i in range(0, min(s + w, n)):  # before that every earlier key is visible
        assert abs(o[i, 0] - i / 2) < 1e-9


def test_local_window_ge_n_equals_global_bitwise():
    n = 64
    q, k, v = _rand((n, 16), 17), _rand((n, 16), 18), _rand((n, 16), 19)
    rows = np.arange(n)
    og, lg = A.attend_masked(q, k, v, A.visibility_mask(W.GLOBAL, 0, 0, None, rows, n), 0.3)
    ol, ll = A.attend_masked(q, k, v, A.visibility_mask(W.LOCAL, 2, n, None, rows, n), 0.3)
    assert np.array_equal(og, ol) and np.array_equal(lg, ll)


def test_perturbing_invisible_keys_changes_nothing():
    n, s, w = 120, 4, 20
    q, k, v = _rand((n, 16), 20), _rand((n, 16), 21), _rand((n, 16), 22)
    rows = np.arange(60, n)  # rows whose windows start after the sink
    mask = A.visibility_mask(W.LOCAL, s, w, None, rows, n)
    o1, l1 = A.attend_masked(q[rows], k, v, mask, 0.3)
    never = ~mask.any(axis=0)
    k2, v2 = k.copy(), v.copy()
    k2[never] += 100.0
    v2[never] -= 50.0
    o2, l2 = A.attend_masked(q[rows], k2, v2, mask, 0.3)
    assert never.sum() > 30
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("case", CASES[:4])
def test_softmax_weights_sum_to_one(case):
    kind, s, w, r = case
    n = 50
    q, k, v = _rand((n, 8), 23), _rand((n, 8), 24), _rand((n, 8), 25)
    rows = np.arange(n)
    mask = A.visibility_mask(kind, s, w, r, rows, n)
    _, lse = A.attend_masked(q, k, v, mask, 0.4)
    sc = 0.4 * q @ k.T
    for i in range(n):
        if mask[i].any():
            assert abs(np.exp(sc[i, mask[i]] - lse[i]).sum() - 1.0) < 1e-12


def test_retrieval_special_cases():
    n, d = 40, 8
    q, k, v = _rand((n, d), 26), _rand((n, d), 27), _rand((n, d), 28)
    rows = np.arange(n)
    # |R| = 1: rows at or after r see exactly v_r; earlier rows see nothing
    o, lse = A.attend_masked(q, k, v, A.visibility_mask(W.RETRIEVAL, 0, 0, [13], rows, n), 0.5)
    assert np.array_equal(o[13:], np.repeat(v[13:14], n - 13, axis=0))
    assert np.all(o[:13] == 0) and np.all(np.isneginf(lse[:13]))
    # R = everything: same as GLOBAL
    og, lg = A.attend_masked(q, k, v, A.visibility_mask(W.GLOBAL, 0, 0, None, rows, n), 0.5)
    oa, la = A.attend_masked(q, k, v, A.visibility_mask(W.RETRIEVAL, 0, 0, np.arange(n), rows, n), 0.5)
    assert np.array_equal(og, oa) and np.array_equal(lg, la)
    # R empty: O = 0, LSE = -inf everywhere
    oe, le = A.attend_masked(q, k, v, A.visibility_mask(W.RETRIEVAL, 0, 0, [], rows, n), 0.5)
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def test_gqa_grouping_golden():
    g = json.load(open(os.path.join(GOLDEN, "gqa_grouping.json")))
    hq, hk = g["num_q_heads"], g["num_kv_heads"]
    spec = W.Spec(name="gqa", num_layers=1, num_q_heads=hq, num_kv_heads=hk, head_dim=8,
                  page_size=8, seq_len=[24], first_query_pos=[0], kind=[W.GLOBAL] * hk,
                  sink=[0] * hk, window=[1] * hk)
    qb = W.q_bits(spec, 0, seed=5)
    kb, vb = W.kv_bits(spec, 0, seed=5)
    o, _ = A.attention(spec, 0, qb, kb, vb)
    for h in range(hk):
        kb2, vb2 = kb.copy(), vb.copy()
        kb2[:, h] ^= 0x0100  # perturb only KV head h
        vb2[:, h] ^= 0x0100
        o2, _ = A.attention(spec, 0, qb, kb2, vb2)
        changed = [not np.array_equal(o[:, j], o2[:, j]) for j in range(hq)]
        expect = [kv == h for kv in g["kv_head_of_q_head"]]
        assert changed == expect


def test_decode_row_equals_last_prefill_row():
    pre = W.tiny("prefill", n=97)
    dec = W.decode_form(pre)
    kb, vb = W.kv_bits(pre, 0)
    qb = W.q_bits(pre, 0)
    o_p, l_p = A.attention(pre, 0, qb, kb, vb)
    o_d, l_d = A.attention(dec, 0, qb[-1:], kb, vb)
    # equal in exact arithmetic; BLAS may order a 1-row product's sums differently
    assert np.max(np.abs(o_p[-1:] - o_d)) < 1e-12 and np.max(np.abs(l_p[-1:] - l_d)) < 1e-12


def test_sequences_are_independent():
    spec = W.Spec(name="two", num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=16,
                  page_size=16, seq_len=[33, 50], first_query_pos=[0, 10],
                  kind=[W.GLOBAL, W.LOCAL], sink=[2, 2], window=[8, 8])
    kb, vb = W.kv_bits(spec, 0)
    qb = W.q_bits(spec, 0)
    o, _ = A.attention(spec, 0, qb, kb, vb)
    kb2 = kb.copy()
    kb2[:33] ^= 0x0040  # change sequence 0 only
    o2, _ = A.attention(spec, 0, qb, kb2, vb)
    assert not np.array_equal(o[:33], o2[:33])
    assert np.array_equal(o[33:], o2[33:])
    # the rows of sequence 1 are its positions 10..49, checked against attention_rows
    o_rows, _ = A.attention_rows(spec, 0, 1, np.arange(10, 50), qb[33:], kb[33:], vb[33:])
    assert np.array_equal(o_rows, o[33:])


@pytest.mark.parametrize("n,s,w", [(512, 4, 64), (100, 4, 200), (300, 0, 7), (9, 4, 2), (1000, 10, 33)])
def test_visible_pairs_closed_forms(n, s, w):
    assert A.visible_pairs(W.GLOBAL, 0, 0, None, n) == n * (n + 1) // 2
    a = min(n, s + w)
    assert A.visible_pairs(W.LOCAL, s, w, None, n) == a * (a + 1) // 2 + max(0, n - s - w) * (s + w)


def test_tiny_pair_counts():
    # per Q head over the 512 prefill rows of the tiny workload
    assert A.visible_pairs(W.GLOBAL, 0, 0, None, 512) == 131_328
    assert A.visible_pairs(W.LOCAL, 4, 64, None, 512) == 32_538


def test_bf16_widening_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0], dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = A.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, ref)
