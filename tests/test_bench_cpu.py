"""bench.py's contract, checked without a GPU: the one-GPU refusal, and the shapes of the five
seeded workloads that the bench times and the parity tests run (sizes as the workload
definitions state them: heads, block size, lengths, pool slack, shared prefix)."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""  # no JSON line for a configuration that was not run
    assert "one GPU" in r.stderr


def _common(c: W.Case, bs: int):
    assert (c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size) == (32, 8, 64, bs)
    assert c.scale == 1.0 / 8
    need = -(-c.ctx_lens.astype(np.int64) // bs)  # blocks each sequence uses
    for s in range(c.n_seqs):
        pages = c.block_tables[s, : need[s]]
        assert np.all((pages >= 0) & (pages < c.num_pages))
    return need


def test_workload_1_single_sequence():
    c = W.make_case(1, values=False)
    need = _common(c, 16)
    assert list(c.ctx_lens) == [37] and c.num_pages == 64
    assert len(c.decode_seqs) == 1 and len(c.prefill_seqs) == 0
    assert len(set(c.block_tables[0, : need[0]].tolist())) == need[0]


def test_workload_2_batched_decode():
    c = W.make_case(2, values=False)
    need = _common(c, 16)
    assert c.n_seqs == 64 and len(c.decode_seqs) == 64
    assert c.ctx_lens.min() >= 1 and c.ctx_lens.max() <= 2048
    assert c.num_pages == int(np.ceil(need.sum() * 1.10))  # total pages + 10%
    used = np.concatenate([c.block_tables[s, : need[s]] for s in range(64)])
    assert len(np.unique(used)) == need.sum()  # no page serves two sequences


def test_workload_3_prefill():
    c = W.make_case(3, values=False)
    _common(c, 16)
    assert c.n_seqs == 8 and len(c.prefill_seqs) == 8
    lens = c.q_lens_prefill
    assert np.array_equal(lens, c.ctx_lens)  # whole prompts, no cached context
    assert lens.min() >= 128 and lens.max() <= 1024
    assert 4000 <= lens.sum() <= 5200  # about 4.5k tokens


def test_workload_4_long_context():
    c = W.make_case(4, values=False)
    _common(c, 32)
    assert list(c.ctx_lens) == [32768] * 16
    assert c.sigma_kv == 0.5
    assert c.kv_tokens() * 2 * 8 * 64 * 2 == 1 << 30  # exactly 1 GiB of K and V


def test_workload_5_mixed_step():
    c = W.make_case(5, values=False)
    need = _common(c, 32)
    assert W.NUM_LAYERS[5] == 16
    dec = c.ctx_lens[c.decode_seqs.start:c.decode_seqs.stop]
    assert len(dec) == 128 and dec.min() >= 16 and dec.max() <= 8192
    (p,) = list(c.prefill_seqs)
    assert (c.ctx_lens[p], c.new_lens[p]) == (1024, 512)  # a 512-token chunk over 512 cached
    assert len(c.shared_seqs) == 32 and c.shared_prefix_tokens == 256
    first = c.block_tables[c.shared_seqs, :8]  # 256 tokens = 8 pages of 32
    assert np.all(first == first[0])
    assert np.all(c.ctx_lens[c.shared_seqs] >= 257)  # the shared pages are never appended to
    others = [s for s in range(c.n_seqs) if s not in set(c.shared_seqs.tolist())]
    assert not set(first[0].tolist()) & set(
        np.concatenate([c.block_tables[s, : need[s]] for s in others]).tolist())


def test_reported_byte_counts():
    """The unique-KV and minimum-prefill-traffic figures printed beside the algorithmic ones:
    in the 16-layer mixed step 32 decode sequences read one 256-token prefix, so 31 x 256
    tokens x 2048 B fewer unique bytes; the 8-prompt prefill moves q and out once (ΣL rows x
    4096 B each) and K/V once (ΣL x 2048 B)."""
    sys.path.insert(0, ROOT)
    import bench

    c5 = W.make_case(5, values=False)
    assert c5.kv_tokens() * 2048 - bench.unique_kv_bytes(c5) == 31 * 256 * 2048
    c3 = W.make_case(3, values=False)
    total = int(c3.ctx_lens.sum())
    assert bench.prefill_min_bytes(c3) == total * (2 * 4096 + 2048)
    for cfg in (2, 4):
        c = W.make_case(cfg, values=False)
        assert bench.unique_kv_bytes(c) == c.kv_tokens() * 2048  # nothing shared
