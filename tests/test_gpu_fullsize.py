"""Parity at the full sizes of the five workloads and the bf16 baseline, on sampled outputs.

Each test fills the whole cache on the GPU through the C ABI and decodes it
in the launch configuration the benchmark times (default split planner, work
sharing on). The oracle then rebuilds, from the same input tensors, the cache
of a few sampled (sequence, KV head) units (a one-head layout with that
head's bits) and computes their attention. Compared:
- the GPU output rows of those units against the oracle (max relative error
  per output vector at most 2e-3);
- a sample of stored code rows and metadata of those units against the
  oracle's rows (identical except codes off by one at rounding ties, at a
  rate of at most 1e-5).
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
from quantized_decode_attention_03_amd import kvq, synth
from tests import kvq_testlib as T

pytestmark = pytest.mark.gpu

TIE_RATE = 1e-5
ROW_SAMPLE = 512
ORACLE_THREADS = 8  # oracle units computed side by side (numpy releases the GIL in its array work)


def device_rows(pool, block_bytes, table_np, seq, positions, area_off, d, bits):
    """Stored bytes (and meta) of the given tokens of one head area, gathered on the device."""
    rb = d * bits // 8
    pos = np.asarray(positions)
    blk = torch.from_numpy(table_np[seq, pos // 16].astype(np.int64)).to(pool.device)
    slot = torch.from_numpy(pos % 16).to(pool.device)
    cols = area_off + slot[:, None] * rb + torch.arange(rb, device=pool.device)[None, :]
    rows = pool[blk[:, None], cols].cpu().numpy()
    meta = None
    if bits != 16:
        mcols = area_off + 16 * rb + slot[:, None] * 8 + torch.arange(8, device=pool.device)[None, :]
        meta = pool[blk[:, None], mcols].cpu().numpy().copy().view(np.float32).reshape(-1, 2)
    return rows, meta


def oracle_unit(k_rows, v_rows, q_rows, bk, bv, n):
    """The oracle's cache and attention for one (sequence, KV head) unit.

    k_rows, v_rows: [T, d] float32 (bf16 values); q_rows: [G, d]."""
    t, d = k_rows.shape
    g = q_rows.shape[0]
    lay = O.Layout(1, g, d, n, [bk], [bv])
    pages = -(-t // 16)
    table = np.arange(pages, dtype=np.int32)[None]
    pool = np.zeros((pages, lay.block_bytes), np.uint8)
    O.quantize_append(lay, pool, table, np.array([0]), k_rows[None, :, None, :], v_rows[None, :, None, :])
    return lay, pool, table


def check_unit_rows(L, gpu_pool, gpu_table, b, h, lay, ref_pool, ref_table, k_rows, v_rows, positions, stats):
    d, n = L.head_dim, L.had_block
    for x, bits, goff, roff in ((k_rows, L.bits_k[h], L.k_off[h], lay.k_off[0]),
                                (v_rows, L.bits_v[h], L.v_off[h], lay.v_off[0])):
        g_rows, g_meta = device_rows(gpu_pool, L.block_bytes, gpu_table, b, positions, goff, d, bits)
        r_rows, r_meta = T.gather_rows(ref_pool, lay.block_bytes, ref_table, 0, positions, roff, d, bits)
        T.compare_rows(g_rows, g_meta, r_rows, r_meta, O.rotate(x[positions], n), bits, d, stats)


def full_cache(L, batch, tokens, k, v, seed):
    """Pool and permuted page table for `batch` sequences of `tokens`, filled in one append."""
    pages = -(-tokens // 16)
    n_blocks = batch * pages
    table = np.full((batch, pages), -1, np.int32)
    kvq.kvq_page_alloc(synth.free_list(n_blocks, seed), 0, np.zeros(batch, np.int32),
                       np.full(batch, tokens, np.int32), table)
    pool = torch.empty((n_blocks, L.block_bytes), dtype=torch.uint8, device=T.DEV)
    table_t = torch.from_numpy(table).to(T.DEV)
    kvq.kvq_quantize_append(L, pool, table_t, torch.zeros(batch, dtype=torch.int32, device=T.DEV), k, v)
    return pool, table, table_t


def decode_units(L, pool, table_t, batch, tokens, q):
    lens = torch.full((batch,), tokens, dtype=torch.int32, device=T.DEV)
    return kvq.kvq_decode_attn([kvq.Segment(L, pool, table_t, lens, tokens)], q).cpu().numpy()


def run_units(L, pool, table, out, k, v, q, units, seed, all_rows=()):
    """Oracle comparison for the sampled units; returns the code statistics.

    Units listed in all_rows have every stored row compared, the others a
    sample of ROW_SAMPLE rows."""
    g, n = L.group, L.had_block
    rng = np.random.default_rng(seed)
    stats = T.CodeStats()
    tokens = k.shape[1]
    for b, h in units:
        k_rows = k[b, :, h].float().cpu().numpy()
        v_rows = v[b, :, h].float().cpu().numpy()
        q_rows = q[b, h * g:(h + 1) * g].float().cpu().numpy()
        lay, ref_pool, ref_table = oracle_unit(k_rows, v_rows, q_rows, L.bits_k[h], L.bits_v[h], n)
        expect = O.decode_attention([(lay, ref_pool, ref_table, np.array([tokens]))],
                                    q_rows[None].astype(np.float64))[0]
        err = T.max_rel_err(out[b, h * g:(h + 1) * g], expect)
        assert err <= T.ATTN_TOL, f"unit (b={b}, h={h}): max relative error {err:.3e}"
        if (b, h) in all_rows:
            positions = np.arange(tokens)
        else:
            positions = np.sort(rng.choice(tokens, size=min(ROW_SAMPLE, tokens), replace=False))
        check_unit_rows(L, pool, table, b, h, lay, ref_pool, ref_table, k_rows, v_rows, positions, stats)
    assert stats.rate <= TIE_RATE
    return stats


def run_units_threaded(L, pool, table, out, k, v, q, units, seed, all_rows=(), row_sample=ROW_SAMPLE):
    """run_units with the oracle's per-unit work on ORACLE_THREADS threads.

    Inputs are copied to the host and the GPU rows gathered in the calling
    thread; the threads run only the oracle (numpy)."""
    g, n = L.group, L.had_block
    tokens = k.shape[1]
    inputs = [(k[b, :, h].float().cpu().numpy(), v[b, :, h].float().cpu().numpy(),
               q[b, h * g:(h + 1) * g].float().cpu().numpy()) for b, h in units]

    def oracle(i):
        (b, h), (k_rows, v_rows, q_rows) = units[i], inputs[i]
        lay, ref_pool, ref_table = oracle_unit(k_rows, v_rows, q_rows, L.bits_k[h], L.bits_v[h], n)
        expect = O.decode_attention([(lay, ref_pool, ref_table, np.array([tokens]))],
                                    q_rows[None].astype(np.float64))[0]
        return lay, ref_pool, ref_table, expect

    rng = np.random.default_rng(seed)
    stats = T.CodeStats()
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        for i, (lay, ref_pool, ref_table, expect) in enumerate(ex.map(oracle, range(len(units)))):
            b, h = units[i]
            err = T.max_rel_err(out[b, h * g:(h + 1) * g], expect)
            assert err <= T.ATTN_TOL, f"unit (b={b}, h={h}): max relative error {err:.3e}"
            if (b, h) in all_rows:
                positions = np.arange(tokens)
            else:
                positions = np.sort(rng.choice(tokens, size=min(row_sample, tokens), replace=False))
            k_rows, v_rows, _ = inputs[i]
            check_unit_rows(L, pool, table, b, h, lay, ref_pool, ref_table, k_rows, v_rows, positions, stats)
            inputs[i] = None
    assert stats.rate <= TIE_RATE
    return stats


@pytest.fixture(scope="module")
def llama32k():
    """One layer of the 32k workload, filled and decoded as the benchmark runs it."""
    batch, tokens, hkv, group, d = 16, 32768, 8, 4, 128
    L = kvq.kvq_layout_init(hkv, group, d, 128, [4] * hkv, [4] * hkv)
    k, v, q = synth.llama_layer_torch(2000, batch, tokens, hkv, group, d, device=T.DEV)
    pool, table, table_t = full_cache(L, batch, tokens, k, v, seed=2000)
    out = decode_units(L, pool, table_t, batch, tokens, q)
    yield L, pool, table, out, k, v, q
    del k, v, q, pool, table_t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(4))
def test_llama_32k_decode_full_size(llama32k, part):
    """Batch 16, 32768 tokens, 8 KV heads x 4, head_dim 128, K4/V4, Hadamard 128 (one layer).

    Every one of the 128 (sequence, KV head) units is compared against the
    oracle, 32 per part (sequences 4*part to 4*part + 3). Units of sequence 0
    have every stored row compared, the others 128 sampled rows."""
    L, pool, table, out, k, v, q = llama32k
    assert np.all(np.isfinite(out))
    units = [(b, h) for b in range(4 * part, 4 * part + 4) for h in range(L.num_kv_heads)]
    run_units_threaded(L, pool, table, out, k, v, q, units, seed=1 + part,
                       all_rows={(0, h) for h in range(L.num_kv_heads)}, row_sample=128)


def test_bf16_32k_baseline_decode_full_size():
    """The unquantized baseline at the 32k shape: bf16 rows (rotated, no metadata), batch 16, one layer."""
    batch, tokens, hkv, group, d = 16, 32768, 8, 4, 128
    L = kvq.kvq_layout_init(hkv, group, d, 128, [16] * hkv, [16] * hkv)
    k, v, q = synth.llama_layer_torch(2001, batch, tokens, hkv, group, d, device=T.DEV)
    pool, table, table_t = full_cache(L, batch, tokens, k, v, seed=2001)
    out = decode_units(L, pool, table_t, batch, tokens, q)
    assert np.all(np.isfinite(out))
    run_units(L, pool, table, out, k, v, q, [(0, 1), (11, 4), (15, 7)], seed=4)


def test_per_channel_keys_32k_decode_full_size():
    """The 32k shape with keys quantized per channel over each 16-token block (K4) and values per token (V4)."""
    batch, tokens, hkv, group, d = 16, 32768, 8, 4, 128
    L = kvq.kvq_layout_init(hkv, group, d, 128, [4] * hkv, [4] * hkv, key_per_channel=True)
    k, v, q = synth.llama_layer_torch(2002, batch, tokens, hkv, group, d, device=T.DEV)
    pool, table, table_t = full_cache(L, batch, tokens, k, v, seed=2002)
    out = decode_units(L, pool, table_t, batch, tokens, q)
    assert np.all(np.isfinite(out))
    for b, h in [(0, 0), (13, 6)]:
        k_rows = k[b, :, h].float().cpu().numpy()
        v_rows = v[b, :, h].float().cpu().numpy()
        q_rows = q[b, h * group:(h + 1) * group].float().cpu().numpy()
        lay = O.Layout(1, group, d, 128, [4], [4], key_per_channel=True)
        ref_table = np.arange(tokens // 16, dtype=np.int32)[None]
        ref_pool = np.zeros((tokens // 16, lay.block_bytes), np.uint8)
        O.quantize_append(lay, ref_pool, ref_table, np.array([0]), k_rows[None, :, None, :], v_rows[None, :, None, :])
        expect = O.decode_attention([(lay, ref_pool, ref_table, np.array([tokens]))],
                                    q_rows[None].astype(np.float64))[0]
        err = T.max_rel_err(out[b, h * group:(h + 1) * group], expect)
        assert err <= T.ATTN_TOL, f"unit (b={b}, h={h}): max relative error {err:.3e}"


def test_mixed_precision_32k_decode_full_size():
    """Batch 8, 32768 tokens, per-head bits from kvq_plan_bits (average 3, ladder {2,3,4,8}).

    As the benchmark runs it: several layers decoded one after another through
    one workspace sized for the largest of them, so layers with different
    split plans (those with an 8-bit head plan fewer splits) reuse the
    workspace. Layers decoded: every layer with an 8-bit head, the layer with
    the most distinct (K, V) pairs, and the layers next to them; one unit per
    distinct pair of each is compared against the oracle."""
    batch, tokens, hkv, group, d, layers = 8, 32768, 8, 4, 128, 32
    ladder = [2, 3, 4, 8]
    w_k = synth.sensitivities(layers, hkv, seed=3).ravel()
    w_v = synth.sensitivities(layers, hkv, seed=33).ravel()
    budget = 3 * layers * hkv
    bits_k = kvq.kvq_plan_bits(w_k, 1.0, 3.6, ladder, budget)[0].reshape(layers, hkv)
    bits_v = kvq.kvq_plan_bits(w_v, 1.0, 5.3, ladder, budget)[0].reshape(layers, hkv)
    ref_k, left_k = O.plan_bits_greedy(w_k.astype(np.float32), 1.0, 3.6, ladder, budget)
    assert left_k == 0 and np.array_equal(bits_k.ravel(), np.asarray(ref_k))
    wide = [l for l in range(layers) if (bits_k[l] == 8).any() or (bits_v[l] == 8).any()]
    pairs = [len({(int(a), int(c)) for a, c in zip(bits_k[l], bits_v[l])}) for l in range(layers)]
    most = int(np.argmax(pairs))
    chosen = sorted({most, *wide, *(l + 1 for l in wide if l + 1 < layers), (most + 1) % layers})
    assert wide, "the planner was expected to give some head 8 bits"
    built = []
    for layer in chosen:
        bk, bv = [int(x) for x in bits_k[layer]], [int(x) for x in bits_v[layer]]
        L = kvq.kvq_layout_init(hkv, group, d, 128, bk, bv)
        k, v, q = synth.llama_layer_torch(3000 + layer, batch, tokens, hkv, group, d, device=T.DEV)
        pool, table, table_t = full_cache(L, batch, tokens, k, v, seed=3000 + layer)
        lens = torch.full((batch,), tokens, dtype=torch.int32, device=T.DEV)
        built.append((layer, L, pool, table, [kvq.Segment(L, pool, table_t, lens, tokens)], k, v, q))
    sizes = [kvq.kvq_decode_workspace_bytes(seg, batch) for (_, _, _, _, seg, _, _, _) in built]
    assert len(set(sizes)) > 1, "the chosen layers were expected to have different split plans"
    ws = torch.empty(max(sizes), dtype=torch.uint8, device=T.DEV)
    kvq.kvq_decode_workspace_init(ws)
    outs = [kvq.kvq_decode_attn(seg, q, ws=ws).cpu().numpy() for (_, _, _, _, seg, _, _, q) in built]
    for (layer, L, pool, table, _, k, v, q), out in zip(built, outs):
        assert np.all(np.isfinite(out))
        bk, bv = list(L.bits_k[:hkv]), list(L.bits_v[:hkv])
        seen, units = set(), []
        for h in range(hkv):
            if (bk[h], bv[h]) not in seen:
                seen.add((bk[h], bv[h]))
                units.append(((layer + len(units)) % batch, h))
        run_units(L, pool, table, out, k, v, q, units, seed=2 + layer)
    head = ws[:kvq.KVQ_DECODE_COUNTER_BYTES].view(torch.int32).cpu().numpy()
    assert np.all(head == 0)


def test_long_context_131k_three_segments_full_size():
    """Batch 1, 131072 tokens, Hadamard 32: bf16 window of 128, log-spaced 4-bit subset, 2-bit rest.
    Every KV head is compared against the oracle."""
    tokens, window, hkv, group, d = 131072, 128, 8, 4, 128
    cls = kvq.kvq_logquant_classes(tokens, window)
    assert np.array_equal(cls.astype(np.int32), O.logquant_precision_map(tokens, window))
    counts = [int((cls == c).sum()) for c in range(3)]
    assert counts == [128, 1280, 129664]
    k, v, q = synth.llama_layer_torch(4, 1, tokens, hkv, group, d, device=T.DEV)
    segs, keep = [], []
    for c, bits in ((0, 16), (1, 4), (2, 2)):
        idx = torch.from_numpy(np.flatnonzero(cls == c)).to(T.DEV)
        L = kvq.kvq_layout_init(hkv, group, d, 32, [bits] * hkv, [bits] * hkv)
        kk = k[:, idx].contiguous()
        vv = v[:, idx].contiguous()
        pool, table, table_t = full_cache(L, 1, counts[c], kk, vv, seed=40 + c)
        lens = torch.full((1,), counts[c], dtype=torch.int32, device=T.DEV)
        segs.append(kvq.Segment(L, pool, table_t, lens, counts[c]))
        keep.append((L, pool, table, kk, vv))
    out = kvq.kvq_decode_attn(segs, q).cpu().numpy()
    assert np.all(np.isfinite(out))
    for h in range(hkv):
        q_rows = q[0, h * group:(h + 1) * group].float().cpu().numpy()
        ref_segs = []
        stats = T.CodeStats()
        for c, (L, pool, table, kk, vv) in enumerate(keep):
            k_rows = kk[0, :, h].float().cpu().numpy()
            v_rows = vv[0, :, h].float().cpu().numpy()
            lay, ref_pool, ref_table = oracle_unit(k_rows, v_rows, q_rows, L.bits_k[h], L.bits_v[h], 32)
            ref_segs.append((lay, ref_pool, ref_table, np.array([counts[c]])))
            positions = np.sort(np.random.default_rng(c).choice(counts[c], size=min(ROW_SAMPLE, counts[c]),
                                                                replace=False))
            check_unit_rows(L, pool, table, 0, h, lay, ref_pool, ref_table, k_rows, v_rows, positions, stats)
        expect = O.decode_attention(ref_segs, q_rows[None].astype(np.float64))[0]
        err = T.max_rel_err(out[0, h * group:(h + 1) * group], expect)
        assert err <= T.ATTN_TOL, f"head {h}: max relative error {err:.3e}"
        assert stats.rate <= TIE_RATE


def test_bulk_append_16k_then_decode_full_size():
    """Batch 4, 16384 new tokens in one append, K4/V2, Hadamard 128, then one decode over them.
    Every (sequence, KV head) unit is compared against the oracle."""
    batch, tokens, hkv, group, d = 4, 16384, 8, 4, 128
    L = kvq.kvq_layout_init(hkv, group, d, 128, [4] * hkv, [2] * hkv)
    k, v, q = synth.llama_layer_torch(5, batch, tokens, hkv, group, d, device=T.DEV)
    pool, table, table_t = full_cache(L, batch, tokens, k, v, seed=5)
    out = decode_units(L, pool, table_t, batch, tokens, q)
    assert np.all(np.isfinite(out))
    # all 32 units' outputs; sampled stored rows of each
    units = [(b, h) for b in range(batch) for h in range(hkv)]
    run_units_threaded(L, pool, table, out, k, v, q, units, seed=3, row_sample=256)


def test_long_context_three_segments_equal_one_merged_segment():
    """The union over segments is the attention over their tokens in any order (LogQuant page,
    Methodology 4, A.V = A_P.V_P): the 131072 tokens at one width (2 bits) as one segment, and the same
    tokens split by the long-context classes into three segments of that width, decode to the same
    output (up to the order of the fp32 sums)."""
    tokens, window, hkv, group, d = 131072, 128, 8, 4, 128
    cls = kvq.kvq_logquant_classes(tokens, window)
    k, v, q = synth.llama_layer_torch(44, 1, tokens, hkv, group, d, device=T.DEV)
    L = kvq.kvq_layout_init(hkv, group, d, 32, [2] * hkv, [2] * hkv)
    pool, _, table_t = full_cache(L, 1, tokens, k, v, seed=45)
    one = kvq.kvq_decode_attn([kvq.Segment(L, pool, table_t, torch.full((1,), tokens, dtype=torch.int32,
                                                                         device=T.DEV), tokens)], q)
    segs = []
    for c in range(3):
        idx = torch.from_numpy(np.flatnonzero(cls == c)).to(T.DEV)
        n = int(idx.numel())
        p, _, t = full_cache(L, 1, n, k[:, idx].contiguous(), v[:, idx].contiguous(), seed=46 + c)
        segs.append(kvq.Segment(L, p, t, torch.full((1,), n, dtype=torch.int32, device=T.DEV), n))
    three = kvq.kvq_decode_attn(segs, q)
    assert T.max_rel_err(three.cpu().numpy(), one.cpu().numpy()) < 1e-5
