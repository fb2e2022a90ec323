"""Parity of the HIP library against the CPU oracle on the GPU (marked ``gpu``).

Every output is compared element by element with the oracle on the same seeded inputs:
bf16 outputs widened to fp32 against the fp64 oracle rounded to fp32, max-abs <= 1e-2
and mean-abs <= 1e-3; kv_append must reproduce the oracle's pools bit for bit (sentinel
bytes included).  The two full-size workloads (16 x 32768 decode; two layers of the
mixed step) are checked on every row, in the launch configuration the bench uses.
Elements with |oracle| >= 4, where half a bf16 unit exceeds 1e-2, are held to half a bf16
unit and counted (``tests.helpers.parity_stats``)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import GpuCase, assert_close, bits_host
from tests.helpers import oracle_decode, oracle_pools, oracle_prefill

pytestmark = pytest.mark.gpu


def torch_index(ids):
    import torch

    return torch.as_tensor(ids, dtype=torch.long, device="cuda:0")


def _announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


# ---------------------------------------------------------------------------------------
# kv_append: bit exact
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_kv_append_bit_exact_workloads(cfg):
    case = W.make_case(cfg)
    _announce(f"kv_append workload {cfg}")
    g = GpuCase(case)
    kp, vp = oracle_pools(case)
    assert np.array_equal(bits_host(g.kp), kp)
    assert np.array_equal(bits_host(g.vp), vp)


@pytest.mark.parametrize("bs", [16, 32])
def test_kv_append_bit_exact_ragged(bs):
    case = W.custom_case([1, 31, 32, 33, 100, 7], [1, 31, 5, 33, 64, 2], kind="prefill",
                         block_size=bs, seed=40 + bs)
    _announce(f"kv_append ragged bs={bs}")
    g = GpuCase(case)
    kp, vp = oracle_pools(case)
    assert np.array_equal(bits_host(g.kp), kp)
    assert np.array_equal(bits_host(g.vp), vp)


# ---------------------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2])
def test_decode_workload_parity(cfg):
    case = W.make_case(cfg)
    _announce(f"decode workload {cfg}")
    g = GpuCase(case)
    out = g.decode()
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)
    mx, mean = assert_close(out, ref, f"decode cfg{cfg}")
    _announce(f"decode workload {cfg}: max-abs {mx:.2e} mean-abs {mean:.2e}")


SWEEP_CTX = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 255, 256, 257, 300, 511, 512, 513,
             1000, 1025]


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("part", [0, 64, 256, 512])
def test_decode_length_sweep(bs, part):
    case = W.custom_case(SWEEP_CTX, [1] * len(SWEEP_CTX), block_size=bs, seed=50 + bs)
    _announce(f"decode sweep bs={bs} part={part}")
    g = GpuCase(case)
    out = g.decode(partition_tokens=part)
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)
    assert_close(out, ref, f"sweep bs={bs} part={part}")


@pytest.mark.parametrize("part", [0, 128])
def test_decode_many_sequences(part):
    """700 sequences: the device-side prefix sum gives each of its 256 chunks three
    sequences; workers start and end inside and across sequences."""
    rng = np.random.default_rng(64)
    ctx = rng.integers(1, 200, size=700, endpoint=True)
    case = W.custom_case(ctx, [1] * 700, block_size=32, seed=64)
    _announce(f"decode 700 sequences part={part}")
    g = GpuCase(case)
    out = g.decode(partition_tokens=part)
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)
    assert_close(out, ref, f"700 sequences part={part}")


def test_decode_beyond_16k_sequences_sampled():
    """17000 sequences: each of the 256 prefix-sum chunks holds 67 sequences, so a worker
    looking for its first sequence walks more than one block of 64.  Most contexts are
    short (one tile); a few long ones are cut between workers."""
    rng = np.random.default_rng(65)
    n = 17000
    ctx = rng.integers(4, 16, size=n, endpoint=True)
    long_ids = [3, 66, 67, 130, 4000, 8191, 8192, 16999]
    for i, s_ in enumerate(long_ids):
        ctx[s_] = 150 + 97 * i
    case = W.custom_case(ctx, [1] * n, block_size=16, seed=65)
    _announce("decode 17000 sequences, sampled")
    g = GpuCase(case)
    out = g.decode(partition_tokens=64)
    kp, vp = oracle_pools(case)
    picks = sorted(set(long_ids + [0, 1, 2, 63, 64, 65, 68, 133, 134, 255, 256, 9000,
                                   16934, 16998] + list(rng.integers(0, n, size=40))))
    ref = oracle_decode(case, kp, vp, seqs=picks)
    # the tolerance applies to the sampled rows together, as it does to a whole workload
    # (a lone short context sits at the bf16 output-rounding floor of ~1e-3 mean-abs)
    idx = torch_index(picks)
    mx, mean = assert_close(out[idx], ref[picks], "17000 sequences (sampled rows)")
    _announce(f"17000 sequences: max-abs {mx:.2e} mean-abs {mean:.2e}")
    assert np.isfinite(out.float().cpu().numpy()).all()


@pytest.mark.parametrize("heads", [(4, 1), (8, 2), (64, 16)])
@pytest.mark.parametrize("part", [0, 128])
def test_decode_other_head_counts(heads, part):
    hq, hkv = heads
    case = W.custom_case([1, 70, 300, 1025, 64, 65], [1] * 6, block_size=16, seed=66 + hq,
                         num_q_heads=hq, num_kv_heads=hkv)
    _announce(f"decode heads {hq}/{hkv} part={part}")
    g = GpuCase(case)
    out = g.decode(partition_tokens=part)
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)
    assert_close(out, ref, f"heads {hq}/{hkv} part={part}")


def test_decode_empty_context_and_loose_max_ctx():
    case = W.custom_case([0, 5, 0, 40], [0, 1, 0, 1], block_size=16, seed=60)
    _announce("decode empty contexts")
    g = GpuCase(case)
    kp, vp = oracle_pools(case)
    ref = oracle_decode(case, kp, vp)
    for part in (0, 256):
        out = g.decode(partition_tokens=part, max_ctx=case.max_blocks * 16)
        assert_close(out, ref, "empty contexts")
        assert np.all(bits_host(out[0]) == 0) and np.all(bits_host(out[2]) == 0)


def test_decode_context_one_returns_v_exactly():
    case = W.custom_case([1, 1, 1], [1, 1, 1], block_size=32, seed=61, sigma_q=4.0)
    _announce("decode ctx=1")
    g = GpuCase(case)
    out = bits_host(g.decode())
    for s in range(3):
        v0 = case.v_new[case.cu_new_lens[s]]  # [Hkv, d] bits
        for h in range(32):
            assert np.array_equal(out[s, h], v0[h // 4])


def test_decode_page_permutation_shared_prefix_and_determinism():
    case = W.custom_case([300, 97, 33, 800], [1, 1, 1, 1], block_size=16, seed=62,
                         shared_seqs=[0, 3], shared_prefix_tokens=32, slack=1.0)
    _announce("decode invariants")
    g = GpuCase(case)
    ref = bits_host(g.decode(partition_tokens=256))
    assert np.array_equal(ref, bits_host(g.decode(partition_tokens=256)))  # run to run
    # physical page permutation with the block table rewritten: bit-identical
    perm = np.random.default_rng(5).permutation(case.num_pages)
    kp_h, vp_h = bits_host(g.kp), bits_host(g.vp)
    kp2, vp2 = np.empty_like(kp_h), np.empty_like(vp_h)
    kp2[perm] = kp_h
    vp2[perm] = vp_h
    import torch

    from tests.gpu_helpers import bf16_dev, i32_dev
    g.kp.copy_(bf16_dev(kp2))
    g.vp.copy_(bf16_dev(vp2))
    g.dec_bt = i32_dev(perm[case.block_tables])
    assert np.array_equal(ref, bits_host(g.decode(partition_tokens=256)))
    # shared prefix pages vs private copies of the same bytes: bit-identical
    bt = perm[case.block_tables].copy()
    used = set(bt.ravel().tolist())
    free = [p for p in range(case.num_pages) if p not in used]
    for b in range(2):
        src = bt[3, b]
        g.kp[free[b]].copy_(g.kp[src])
        g.vp[free[b]].copy_(g.vp[src])
        bt[3, b] = free[b]
    g.dec_bt = i32_dev(bt)
    torch.cuda.synchronize()
    assert np.array_equal(ref, bits_host(g.decode(partition_tokens=256)))


def test_decode_zero_query_is_mean_of_v():
    case = W.custom_case([200, 5], [1, 1], block_size=32, seed=63)
    case.q_decode[:] = 0
    g = GpuCase(case)
    out = g.decode()
    for s in range(2):
        _, vl = case.logical_kv(s)
        mean = O.bf16_to_f64(vl).mean(axis=0)
        ref = np.repeat(mean, 4, axis=0)[None]
        assert_close(out[s:s + 1], ref, "q=0")


def test_decode_long_context_workload():
    """16 x 32768 tokens, block size 32, split-K with the automatic partition: every
    sequence, every head."""
    case = W.make_case(4)
    _announce("decode workload 4 (16 x 32768), all sequences")
    g = GpuCase(case)
    out = g.decode()
    kp_h, vp_h = bits_host(g.kp), bits_host(g.vp)
    refs = []
    for s in range(16):
        kl, vl = case.logical_kv(s)
        # the library's pool holds exactly the logical rows (layout read by the oracle)
        kb, vb = O.gather(kp_h, vp_h, case.block_tables[s], 32768, 32, 8, 64)
        assert np.array_equal(kb, kl) and np.array_equal(vb, vl)
        refs.append(O.attention(O.bf16_to_f64(case.q_decode[s:s + 1]), O.bf16_to_f64(kl),
                                O.bf16_to_f64(vl), [32768], case.scale))
    mx, mean = assert_close(out, np.concatenate(refs), "cfg4 all sequences")
    _announce(f"cfg4: max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("bs", [16, 32])
def test_decode_one_very_long_sequence(bs):
    """One 131072-token sequence beside a 5-token one, automatic partition: each of the long
    sequence's 8 segments (2048 tiles) is cut over about 128 workers, so the merge combines
    that many partials per row; every head of both sequences against the oracle."""
    ctx = [131072, 5]
    case = W.custom_case(ctx, [1, 1], block_size=bs, seed=130 + bs)
    _announce(f"decode 1 x 131072 + 1 x 5, bs={bs}")
    g = GpuCase(case)
    out = g.decode()
    refs = []
    for s, n in enumerate(ctx):
        kl, vl = case.logical_kv(s)
        refs.append(O.attention(O.bf16_to_f64(case.q_decode[s:s + 1]), O.bf16_to_f64(kl),
                                O.bf16_to_f64(vl), [n], case.scale))
    mx, mean = assert_close(out, np.concatenate(refs), f"1 x 131072, bs {bs}")
    _announce(f"1 x 131072 bs={bs}: max-abs {mx:.2e} mean-abs {mean:.2e}")


# ---------------------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------------------
def test_prefill_workload_parity():
    case = W.make_case(3)
    _announce("prefill workload 3")
    g = GpuCase(case)
    out = g.prefill()
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp)
    mx, mean = assert_close(out, ref, "prefill cfg3")
    _announce(f"prefill workload 3: max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_prefill_chunk_behind_30k_prefix():
    """A 256-token chunk behind a 29,744-token cached prefix (about 470 key stages per
    tile) beside a short prompt, block size 32: the automatic plan (four key groups per
    workgroup, each taking every fourth stage) and eight key pieces with their merge, both
    against the oracle."""
    case = W.custom_case([30000, 1200], [256, 37], kind="prefill", block_size=32, seed=140)
    _announce("prefill chunk behind a 30k prefix")
    g = GpuCase(case)
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp)
    for splits in (0, 8):
        out = g.prefill(kv_splits=splits)
        mx, mean = assert_close(out, ref, f"30k prefix, kv_splits {splits}")
        _announce(f"30k prefix kv_splits={splits}: max-abs {mx:.2e} mean-abs {mean:.2e}")


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_chunked_ragged(bs, causal):
    # chunks after a cached prefix, lengths that are not multiples of the 32-row tile,
    # a one-token chunk and a chunk that is a whole prompt
    case = W.custom_case([70, 33, 129, 1, 200, 64], [7, 33, 100, 1, 1, 40], kind="prefill",
                         block_size=bs, seed=70 + bs)
    _announce(f"prefill chunked bs={bs} causal={causal}")
    g = GpuCase(case)
    out = g.prefill(causal=causal)
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp, causal=causal)
    assert_close(out, ref, f"prefill bs={bs} causal={causal}")


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_long_cached_prefix(bs, causal):
    # chunks behind long cached prefixes: a small grid of many stages per tile (the K/V
    # copies and their patches run through 20+ rounds per key group and block-table
    # entries far into the row), contexts that end inside a page, and a one-token chunk
    case = W.custom_case([5000, 3001, 77], [200, 1, 77], kind="prefill", block_size=bs,
                         seed=76 + bs)
    _announce(f"prefill long cached prefix bs={bs} causal={causal}")
    g = GpuCase(case)
    out = g.prefill(causal=causal)
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp, causal=causal)
    assert_close(out, ref, f"prefill long prefix bs={bs} causal={causal}")


@pytest.mark.parametrize("splits", [1, 2, 5, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_key_splits(splits, causal):
    # each tile's keys cut into pieces merged by log-sum-exp (pieces shorter than a stage
    # stay empty), against the same call unsplit and the oracle
    case = W.custom_case([70, 33, 129, 1, 200, 64, 300], [7, 33, 100, 1, 1, 40, 300],
                         kind="prefill", block_size=16, seed=90)
    _announce(f"prefill kv_splits={splits} causal={causal}")
    g = GpuCase(case)
    out = g.prefill(causal=causal, kv_splits=splits)
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp, causal=causal)
    assert_close(out, ref, f"prefill kv_splits={splits} causal={causal}")


SMALL_GRIDS = {
    # 160 tiles (fewer than the compute units): two key groups of four head-waves
    "two-groups": ([70, 33, 129, 1, 640], [7, 33, 100, 1, 96], 32),
    # 80 tiles (at most half the compute units): two workgroups per tile, two head-waves
    # per group, four key groups
    "four-groups": ([70, 33, 129, 1, 640], [7, 33, 60, 1, 50], 16),
}


@pytest.mark.parametrize("grid", sorted(SMALL_GRIDS))
@pytest.mark.parametrize("splits", [1, 2, 5, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_key_groups_and_splits_small_grid(grid, splits, causal):
    # fewer tiles than compute units: key groups per workgroup, merged in LDS, and on top
    # of that the pieces (a piece of fewer stages than groups leaves groups idle)
    ctx, new, bs = SMALL_GRIDS[grid]
    case = W.custom_case(ctx, new, kind="prefill", block_size=bs, seed=92)
    _announce(f"prefill small grid {grid} kv_splits={splits} causal={causal}")
    g = GpuCase(case)
    out = g.prefill(causal=causal, kv_splits=splits)
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp, causal=causal)
    assert_close(out, ref, f"small grid {grid} kv_splits={splits} causal={causal}")


@pytest.mark.parametrize("heads", [(4, 1), (8, 2), (64, 16)])
@pytest.mark.parametrize("bs", [16, 32])
def test_prefill_other_head_counts(heads, bs):
    # one KV head (a tiny grid: two key groups and key pieces), two, and sixteen (a grid of
    # one key group), over prompts and chunks with cached prefixes
    hq, hkv = heads
    case = W.custom_case([300, 37, 129, 64], [300, 20, 65, 1], kind="prefill", block_size=bs,
                         seed=93 + hq + bs, num_q_heads=hq, num_kv_heads=hkv)
    _announce(f"prefill heads {hq}/{hkv} bs={bs}")
    g = GpuCase(case)
    out = g.prefill()
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp)
    assert_close(out, ref, f"prefill heads {hq}/{hkv} bs={bs}")


@pytest.mark.parametrize("splits", [1, 4])
def test_prefill_out_of_range_page_gives_nan_rows(splits):
    # a block-table entry outside the pool: exactly the rows whose keys reach that block
    # come out NaN (every head), the others match the oracle
    case = W.custom_case([200, 90], [200, 90], kind="prefill", block_size=16, seed=91)
    kp, vp = oracle_pools(case)
    ref = oracle_prefill(case, kp, vp)
    g = GpuCase(case)
    bt = case.block_tables.copy()
    blk = 5  # keys 80 .. 95 of sequence 0
    bt[0, blk] = case.num_pages + 3
    from tests.gpu_helpers import i32_dev
    g.pre_bt = i32_dev(bt)
    out_t = g.prefill(kv_splits=splits)
    out = out_t.float().cpu().numpy()
    pos = np.arange(200)  # sequence 0 is a whole prompt: row i sits at position i
    sees = pos >= blk * 16
    assert np.isnan(out[:200][sees]).all()
    assert not np.isnan(out[:200][~sees]).any() and not np.isnan(out[200:]).any()
    ok = np.nonzero(np.concatenate([~sees, np.ones(90, bool)]))[0]
    assert_close(out_t[torch_index(ok)], ref[ok], "rows that do not read the bad page")


def test_prefill_last_row_matches_decode_and_permutation():
    case = W.custom_case([150, 47], [150, 47], kind="prefill", block_size=16, seed=80)
    g = GpuCase(case)
    out = g.prefill()
    ref_bits = bits_host(out)
    assert np.array_equal(ref_bits, bits_host(g.prefill()))  # run to run
    kp, vp = oracle_pools(case)
    cu = case.cu_q_lens_prefill
    for s in range(2):
        dec = O.decode(case.q_prefill[cu[s + 1] - 1:cu[s + 1]], kp, vp, case.block_tables[s:s + 1],
                       [int(case.ctx_lens[s])], 16, 8, 64, case.scale)
        assert_close(out[cu[s + 1] - 1:cu[s + 1]], dec, "last prefill row vs decode")
    perm = np.random.default_rng(9).permutation(case.num_pages)
    kp_h, vp_h = bits_host(g.kp), bits_host(g.vp)
    kp2, vp2 = np.empty_like(kp_h), np.empty_like(vp_h)
    kp2[perm] = kp_h
    vp2[perm] = vp_h
    from tests.gpu_helpers import bf16_dev, i32_dev
    g.kp.copy_(bf16_dev(kp2))
    g.vp.copy_(bf16_dev(vp2))
    g.pre_bt = i32_dev(perm[case.block_tables])
    assert np.array_equal(ref_bits, bits_host(g.prefill()))


# ---------------------------------------------------------------------------------------
# the mixed step, one layer at full size
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("layer", [0, 1])
def test_mixed_step_layer(layer):
    """One layer of the mixed step at full size, in the bench's launch configuration:
    every chunk row and every one of the 128 decode rows against the oracle."""
    case = W.make_case(5, layer=layer)
    _announce(f"mixed step layer {layer} (chunk 512 + 128 decode), all rows")
    g = GpuCase(case)
    dec = g.decode()
    pre = g.prefill()
    # chunk rows: every row, against the oracle over the chunk sequence's logical K/V
    s = case.prefill_seqs.start
    kl, vl = case.logical_kv(s)
    ctx = int(case.ctx_lens[s])
    ql = int(case.new_lens[s])
    vis = [ctx - ql + i + 1 for i in range(ql)]
    ref = O.attention(O.bf16_to_f64(case.q_prefill), O.bf16_to_f64(kl), O.bf16_to_f64(vl), vis,
                      case.scale)
    mx, mean = assert_close(pre, ref, f"mixed chunk layer {layer}")
    _announce(f"mixed chunk layer {layer}: max-abs {mx:.2e} mean-abs {mean:.2e}")
    # decode rows: all 128 (shared-prefix sequences among them), read back through the
    # library's pool, which must hold exactly each sequence's logical rows
    kp_h, vp_h = bits_host(g.kp), bits_host(g.vp)
    refs = []
    for d in range(len(case.decode_seqs)):
        kb, vb = O.gather(kp_h, vp_h, case.block_tables[d], int(case.ctx_lens[d]), 32, 8, 64)
        kl, vl = case.logical_kv(d)
        assert np.array_equal(kb, kl) and np.array_equal(vb, vl)
        refs.append(O.attention(O.bf16_to_f64(case.q_decode[d:d + 1]), O.bf16_to_f64(kl),
                                O.bf16_to_f64(vl), [int(case.ctx_lens[d])], case.scale))
    mx, mean = assert_close(dec, np.concatenate(refs), f"mixed decode layer {layer}")
    _announce(f"mixed decode layer {layer}: max-abs {mx:.2e} mean-abs {mean:.2e}")


def test_decode_workspace_needs_no_initialisation():
    """The split-K workspace is scratch: whatever it holds before a call (random bytes, all
    ones, the state another call with other shapes left), and however often it is reused,
    the output is the clean run's, bit for bit."""
    import torch

    import paged_kv_attention_31_amd as pa

    _announce("decode workspace contents")
    case = W.custom_case([700, 1, 3000, 65, 129, 2049], [1] * 6, block_size=32, seed=97)
    other = W.custom_case([5000, 17, 900], [1] * 3, block_size=32, seed=98)
    g, go = GpuCase(case), GpuCase(other)
    c, co = g.case, go.case
    part = 128
    mc, mco = int(c.ctx_lens.max()), int(co.ctx_lens.max())
    nb = max(pa.decode_workspace_bytes(g.geom, len(c.decode_seqs), mc, part),
             pa.decode_workspace_bytes(go.geom, len(co.decode_seqs), mco, part))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda:0")

    def run(gc, mctx):
        out = torch.empty((len(gc.case.decode_seqs), 32, 64), dtype=torch.bfloat16,
                          device="cuda:0")
        pa.decode(gc.geom, out, gc.q_dec, gc.kp, gc.vp, gc.dec_bt, gc.dec_ctx, mctx,
                  gc.case.scale, partition_tokens=part, workspace=ws)
        return bits_host(out)

    ref = bits_host(g.decode(partition_tokens=part))  # its own fresh workspace
    ref_o = bits_host(go.decode(partition_tokens=part))
    assert np.array_equal(run(g, mc), ref)
    ws.copy_(torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda:0"))
    assert np.array_equal(run(g, mc), ref)
    ws.fill_(255)
    assert np.array_equal(run(g, mc), ref)
    for _ in range(3):  # alternating shapes on one workspace
        assert np.array_equal(run(go, mco), ref_o)
        assert np.array_equal(run(g, mc), ref)
