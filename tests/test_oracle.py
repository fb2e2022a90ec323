"""Pins for the CPU oracle: each test checks it against something other than itself
(values the pages fix, closed forms, invariants, brute force).  CPU only."""

from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle as O
import oracle.paged_attention as OP
import workloads as W
from tests.helpers import (brute_force_rows, oracle_decode, oracle_pools, oracle_prefill)

TOL = 1e-12


# ---------------------------------------------------------------------------------------
# values printed on (or fixed by) the pages
# ---------------------------------------------------------------------------------------
def test_page_bytes_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "page_bytes.json")))
    assert O.page_bytes(g["block_size"], g["num_kv_heads"], g["head_dim"]) == g["page_bytes"]
    case = W.make_case(1, values=False)
    assert W.page_elems(case) * 2 == g["page_bytes"]


def test_bf16_widening_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "bf16_values.json")))
    bits = np.array([int(c["bits"], 16) for c in g["cases"]], dtype=np.uint16)
    got = O.bf16_to_f64(bits)
    for c, v in zip(g["cases"], got):
        assert v == c["value"], (c, v)


def test_two_token_closed_form(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "two_token_softmax.json")))
    d = 64
    bf = W.f32_to_bf16_bits
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = g["q0"]
    k = np.zeros((3, 1, d), np.float32)
    v = np.zeros((3, 1, d), np.float32)
    k[1, 0, 0] = 1.0
    k[2, 0, 0] = -1.0
    v[0, 0, 0], v[0, 0, 1] = 1.0, 2.0
    v[1, 0, 1], v[1, 0, 2] = -1.0, 0.5
    v[2, 0, :] = 7.0
    out = O.attention(O.bf16_to_f64(bf(q)), O.bf16_to_f64(bf(k)), O.bf16_to_f64(bf(v)), [2],
                      g["scale"])[0, 0]
    e = g["expected"]
    assert abs(out[0] - e["o0"]) < TOL and abs(out[1] - e["o1"]) < TOL
    assert abs(out[2] - e["o2"]) < TOL and np.all(out[3:] == 0.0)


# ---------------------------------------------------------------------------------------
# brute force on tiny inputs
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("heads", [(32, 8), (4, 1)])
def test_decode_matches_brute_force(bs, heads):
    hq, hkv = heads
    case = W.custom_case([37, 1, 33][: 3 if hq == 4 else 2], [1, 1, 1][: 3 if hq == 4 else 2],
                         block_size=bs, num_q_heads=hq, num_kv_heads=hkv, seed=bs + hq)
    kp, vp = oracle_pools(case)
    got = oracle_decode(case, kp, vp)
    for s in range(case.n_seqs):
        kl, vl = case.logical_kv(s)
        bf = brute_force_rows(case.q_decode[s:s + 1], kl, vl, [int(case.ctx_lens[s])], case.scale)
        assert np.max(np.abs(got[s] - np.array(bf[0]))) < TOL


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("heads,ctx,new", [((4, 1), [40, 17, 5], [40, 9, 5]),
                                           ((32, 8), [19, 6], [19, 3])])
def test_prefill_matches_brute_force(causal, heads, ctx, new):
    hq, hkv = heads
    case = W.custom_case(ctx, new, kind="prefill", block_size=16, num_q_heads=hq,
                         num_kv_heads=hkv, seed=7 + hq)
    kp, vp = oracle_pools(case)
    got = oracle_prefill(case, kp, vp, causal=causal)
    cu = case.cu_q_lens_prefill
    for s in range(case.n_seqs):
        kl, vl = case.logical_kv(s)
        c, ql = int(case.ctx_lens[s]), int(case.new_lens[s])
        vis = [(c - ql + i + 1) if causal else c for i in range(ql)]
        bf = brute_force_rows(case.q_prefill[cu[s]:cu[s + 1]], kl, vl, vis, case.scale)
        assert np.max(np.abs(got[cu[s]:cu[s + 1]] - np.array(bf))) < TOL


# ---------------------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------------------
def _permute_pages(case, kp, vp, seed):
    perm = np.random.default_rng(seed).permutation(case.num_pages)  # old page p -> perm[p]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    return perm[case.block_tables].astype(np.int32), kp2, vp2


def test_page_permutation_invariance_decode():
    case = W.custom_case([70, 33, 1, 129], [1, 1, 1, 1], block_size=16, seed=3)
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)
    bt2, kp2, vp2 = _permute_pages(case, kp, vp, 11)
    case.block_tables = bt2
    got = oracle_decode(case, kp2, vp2)
    assert np.array_equal(ref, got)


def test_page_permutation_invariance_prefill():
    case = W.custom_case([45, 64], [45, 20], kind="prefill", block_size=32, seed=4)
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp)
    bt2, kp2, vp2 = _permute_pages(case, kp, vp, 12)
    case.block_tables = bt2
    assert np.array_equal(ref, oracle_prefill(case, kp2, vp2))


def test_online_softmax_equals_three_pass():
    case = W.custom_case([300], [1], block_size=32, seed=5, sigma_q=3.0)
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)[0]
    kb, vb = O.gather(kp, vp, case.block_tables[0], 300, 32, 8, 64)
    got = O.online_softmax_attention(O.bf16_to_f64(case.q_decode[0]), O.bf16_to_f64(kb),
                                     O.bf16_to_f64(vb), 300, case.scale)
    assert np.max(np.abs(got - ref)) <= TOL * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("part", [1, 16, 64, 100, 299, 300, 512])
def test_split_merge_equals_three_pass(part):
    case = W.custom_case([300], [1], block_size=16, seed=6, sigma_q=2.0)
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)[0]
    kb, vb = O.gather(kp, vp, case.block_tables[0], 300, 16, 8, 64)
    qf = O.bf16_to_f64(case.q_decode[0])
    m, den, o = O.partition_partials(qf, O.bf16_to_f64(kb), O.bf16_to_f64(vb), 300,
                                     case.scale, part)
    # add an empty partition: it must not change the merge
    m = np.concatenate([m, np.full((1, m.shape[1]), -np.inf)])
    den = np.concatenate([den, np.zeros((1, den.shape[1]))])
    o = np.concatenate([o, np.zeros((1,) + o.shape[1:])])
    got = O.merge_partials(m, den, o)
    assert np.max(np.abs(got - ref)) <= TOL


def test_context_one_returns_v_exactly():
    case = W.custom_case([1, 1], [1, 1], block_size=16, seed=8, sigma_q=5.0)
    kp, vp = oracle_pools(case)
    got = oracle_decode(case, kp, vp)
    for s in range(2):
        v0 = O.bf16_to_f64(case.v_new[case.cu_new_lens[s]])  # [Hkv, d]
        for h in range(32):
            assert np.array_equal(got[s, h], v0[h // 4])


def test_zero_query_gives_mean_of_v():
    case = W.custom_case([57], [1], block_size=16, seed=9)
    case.q_decode[:] = 0
    kp, vp = oracle_pools(case)
    got = oracle_decode(case, kp, vp)[0]
    _, vl = case.logical_kv(0)
    mean = O.bf16_to_f64(vl).mean(axis=0)  # [Hkv, d]
    for h in range(32):
        assert np.max(np.abs(got[h] - mean[h // 4])) < TOL


def test_linearity_in_v():
    case = W.custom_case([90, 5], [1, 1], block_size=32, seed=10)
    kp, vp = oracle_pools(case)
    base = oracle_decode(case, kp, vp)
    a, c = 0.5, 3.0  # exact in bf16: a*v + c is rounded; compare on the widened values
    r = case.decode_seqs
    out = np.zeros_like(base)
    for s in r:
        kb, vb = O.gather(kp, vp, case.block_tables[s], int(case.ctx_lens[s]), 32, 8, 64)
        vf = a * O.bf16_to_f64(vb) + c
        out[s] = O.attention(O.bf16_to_f64(case.q_decode[s:s + 1]), O.bf16_to_f64(kb), vf,
                             [int(case.ctx_lens[s])], case.scale)[0]
    assert np.max(np.abs(out - (a * base + c))) < 1e-11


def test_gqa_group_heads_with_equal_queries_agree():
    case = W.custom_case([77], [1], block_size=16, seed=13)
    for g in range(8):
        case.q_decode[0, 4 * g + 1: 4 * g + 4] = case.q_decode[0, 4 * g]
    kp, vp = oracle_pools(case)
    got = oracle_decode(case, kp, vp)[0]
    for g in range(8):
        for j in range(1, 4):
            assert np.array_equal(got[4 * g + j], got[4 * g])
    assert not np.array_equal(got[0], got[4])


def test_shared_prefix_equals_private_copies():
    shared = W.custom_case([100, 70, 96], [1, 1, 1], block_size=32, seed=14,
                           shared_seqs=[0, 2], shared_prefix_tokens=64, slack=1.0)
    assert np.array_equal(shared.block_tables[0, :2], shared.block_tables[2, :2])
    kp, vp = oracle_pools(shared)
    ref = oracle_decode(shared, kp, vp)
    # private copies: give sequence 2 its own two pages holding the same bytes
    free = [p for p in range(shared.num_pages) if p not in set(shared.block_tables.ravel())]
    kp2, vp2 = kp.copy(), vp.copy()
    bt2 = shared.block_tables.copy()
    for b in range(2):
        src = shared.block_tables[2, b]
        kp2[free[b]] = kp[src]
        vp2[free[b]] = vp[src]
        bt2[2, b] = free[b]
    shared.block_tables = bt2
    assert np.array_equal(ref, oracle_decode(shared, kp2, vp2))


def test_last_prefill_row_equals_decode_and_chunking():
    ctx = [60, 33]
    case = W.custom_case(ctx, ctx, kind="prefill", block_size=16, seed=15)
    kp, vp = oracle_pools(case)
    full = oracle_prefill(case, kp, vp)
    cu = case.cu_q_lens_prefill
    bt = case.block_tables
    # last causal row == decode of the same context
    for s in range(2):
        dec = O.decode(case.q_prefill[cu[s + 1] - 1: cu[s + 1]], kp, vp, bt[s:s + 1],
                       [ctx[s]], 16, 8, 64, case.scale)
        assert np.max(np.abs(dec[0] - full[cu[s + 1] - 1])) < TOL
    # a chunk (the last 25 / 10 tokens, the rest already cached) == those rows of one shot
    tail = [25, 10]
    qs = np.concatenate([case.q_prefill[cu[s + 1] - tail[s]: cu[s + 1]] for s in range(2)])
    cuq = np.array([0, tail[0], tail[0] + tail[1]])
    chunk = O.prefill(qs, kp, vp, bt, cuq, ctx, 16, 8, 64, case.scale, causal=True)
    ref = np.concatenate([full[cu[s + 1] - tail[s]: cu[s + 1]] for s in range(2)])
    assert np.max(np.abs(chunk - ref)) < TOL
    # a non-causal row == decode over the full context
    nc = O.prefill(qs, kp, vp, bt, cuq, ctx, 16, 8, 64, case.scale, causal=False)
    dec0 = O.decode(qs[:1], kp, vp, bt[:1], [ctx[0]], 16, 8, 64, case.scale)
    assert np.max(np.abs(nc[0] - dec0[0])) < TOL


def test_empty_context_row_is_zero():
    case = W.custom_case([0, 5], [0, 1], block_size=16, seed=16)
    kp, vp = oracle_pools(case)
    got = oracle_decode(case, kp, vp)
    assert np.all(got[0] == 0.0) and np.all(np.isfinite(got[1]))


# ---------------------------------------------------------------------------------------
# kv_append
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("bs", [16, 32])
def test_append_gather_round_trip_and_untouched_bytes(bs):
    case = W.custom_case([50, 3, 64, 17], [50, 1, 10, 17], kind="prefill", block_size=bs,
                         seed=17 + bs)
    kp, vp = oracle_pools(case)
    written = 0
    for s in range(case.n_seqs):
        kl, vl = case.logical_kv(s)
        kb, vb = O.gather(kp, vp, case.block_tables[s], int(case.ctx_lens[s]), bs, 8, 64)
        assert np.array_equal(kb, kl) and np.array_equal(vb, vl)
        written += kl.size
    # every byte no append wrote still holds the sentinel (the random bf16 inputs never
    # produce that NaN pattern)
    assert int((kp != W.SENTINEL_BITS).sum()) == written
    assert int((vp != W.SENTINEL_BITS).sum()) == written
    # appended pages only: the sentinel page and the slack pages are untouched
    assert np.all(kp[case.sentinel_page] == W.SENTINEL_BITS)


def test_layout_offsets_cover_a_page_once():
    for bs in (16, 32):
        seen_k = set()
        seen_v = set()
        for g in range(8):
            for s in range(bs):
                for i in range(64):
                    seen_k.add(O.k_offset(g, s, i, bs, 64))
                    seen_v.add(O.v_offset(g, s, i, bs, 64))
        assert seen_k == set(range(bs * 8 * 64)) == seen_v
    # a 16-byte piece of one token's head vector is contiguous in a K page, and one
    # dimension of all slots is contiguous in a V page
    assert O.k_offset(2, 3, 13, 16, 64) == ((2 * 8 + 1) * 16 + 3) * 8 + 5
    assert O.v_offset(2, 3, 13, 16, 64) == (2 * 64 + 13) * 16 + 3


# ---------------------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------------------
def _decode_vs_brute(case) -> float:
    kp, vp = oracle_pools(case)
    got = oracle_decode(case, kp, vp)
    worst = 0.0
    for s in range(case.n_seqs):
        kl, vl = case.logical_kv(s)
        bf = brute_force_rows(case.q_decode[s:s + 1], kl, vl, [int(case.ctx_lens[s])], case.scale)
        worst = max(worst, float(np.max(np.abs(got[s] - np.array(bf[0])))))
    return worst


def _mutated_attention(head_map=None, scale_mult=1.0, vis_shift=0):
    def attention(q, k, v, n_visible, scale):
        r_rows, hq, d = q.shape
        hkv = k.shape[1]
        group = hq // hkv
        out = np.zeros((r_rows, hq, d))
        for r in range(r_rows):
            n = int(n_visible[r]) + vis_shift
            if n <= 0:
                continue
            for h in range(hq):
                g = head_map(h, hkv, group) if head_map else h // group
                x = scale * scale_mult * (k[:n, g, :] @ q[r, h, :])
                w = np.exp(x - np.max(x))
                out[r, h, :] = (w / w.sum()) @ v[:n, g, :]
        return out
    return attention


@pytest.mark.parametrize("mutation", ["scale", "head_map", "mask_off_by_one"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    case = W.custom_case([20, 9], [1, 1], block_size=16, num_q_heads=8, num_kv_heads=2, seed=21)
    assert _decode_vs_brute(case) < TOL
    if mutation == "scale":
        bad = _mutated_attention(scale_mult=8.0)  # forgets the 1/8
    elif mutation == "head_map":
        bad = _mutated_attention(head_map=lambda h, hkv, grp: h % hkv)
    else:
        bad = _mutated_attention(vis_shift=-1)  # drops the newest key
    monkeypatch.setattr(OP, "attention", bad)
    assert _decode_vs_brute(case) > 1e-3


def test_planted_merge_sign_mistake_is_caught():
    case = W.custom_case([200], [1], block_size=16, seed=22, sigma_q=3.0)
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)[0]
    kb, vb = O.gather(kp, vp, case.block_tables[0], 200, 16, 8, 64)
    m, den, o = O.partition_partials(O.bf16_to_f64(case.q_decode[0]), O.bf16_to_f64(kb),
                                     O.bf16_to_f64(vb), 200, case.scale, 64)
    big = m.max(axis=0)
    f = np.exp(big[None] - m)  # wrong sign in the rescale factor
    bad = (o * f[..., None]).sum(0) / (den * f).sum(0)[..., None]
    assert np.max(np.abs(bad - ref)) > 1e-3
    assert np.max(np.abs(O.merge_partials(m, den, o) - ref)) < TOL


def test_planted_layout_mistake_is_caught(monkeypatch):
    case = W.custom_case([40], [40], kind="prefill", block_size=16, seed=23)
    kp, vp = oracle_pools(case)
    # gather reading slots mirrored inside the page no longer returns what was appended
    orig = OP.k_offset
    monkeypatch.setattr(OP, "k_offset", lambda g, s, i, bs, d: orig(g, bs - 1 - s, i, bs, d))
    OP._Offsets._cache.clear()
    try:
        kb, _ = O.gather(kp, vp, case.block_tables[0], 40, 16, 8, 64)
        kl, _ = case.logical_kv(0)
        assert not np.array_equal(kb, kl)
    finally:
        OP._Offsets._cache.clear()


# ---------------------------------------------------------------------------------------
# generator determinism (integer structure and bytes)
# ---------------------------------------------------------------------------------------
def test_generator_is_deterministic():
    a = W.make_case(1)
    b = W.make_case(1)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.q_decode, b.q_decode) and np.array_equal(a.k_setup, b.k_setup)
    assert len(set(a.block_tables[0].tolist())) == 3
    c3 = W.make_case(3, values=False)
    assert c3.ctx_lens.min() >= 128 and c3.ctx_lens.max() <= 1024
    assert abs(int(c3.ctx_lens.sum()) - 4608) < 600
    c5 = W.make_case(5, values=False)
    assert len(c5.shared_seqs) == 32
    assert np.all(c5.block_tables[c5.shared_seqs, :8] == c5.block_tables[c5.shared_seqs[0], :8])
    used = c5.block_tables[:, :].ravel()
    # every page is assigned at most once, except the shared prefix pages
    nb = (c5.ctx_lens + 31) // 32
    ids = np.concatenate([c5.block_tables[s, :nb[s]] for s in range(c5.n_seqs)])
    uniq, counts = np.unique(ids, return_counts=True)
    assert set(uniq[counts > 1].tolist()) == set(c5.block_tables[c5.shared_seqs[0], :8].tolist())
    assert c5.sentinel_page not in set(ids.tolist()) and used.max() < c5.num_pages
