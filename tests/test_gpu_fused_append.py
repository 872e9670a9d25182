"""kvq_append_decode_attn: one decode step (append one token per sequence, then decode) in one call.

It must equal kvq_quantize_append followed by kvq_decode_attn: the stored rows and metadata bit for bit,
the output up to the order of fp32 sums; and both match the oracle (the SAW-INT4 page, sections 2 and 3:
rotate, quantize token-wise, fused with the cache write; decode over the dequantized cache, the LogQuant
page, Methodology 4, for several segments).
"""

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
from quantized_decode_attention_03_amd import kvq, synth
from tests import kvq_testlib as T
from tests.test_gpu_parity import build_case

pytestmark = pytest.mark.gpu

# Fused against separate calls: both are within ~1.8e-5 of the fp64 oracle for 2-, 3- and 8-bit keys
# (4-bit keys: ~5e-6) and differ in the order of their fp32 sums (the shared page order varies from run
# to run, and the new token enters through the merge in fp32 instead of the matrix cores), so they may
# differ by twice that.
SAME = 4e-5


def new_rows(batch, hkv, d, seed, bf16=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((batch, hkv, d)).astype(np.float32) * 2.0 + 0.5
    v = rng.standard_normal((batch, hkv, d)).astype(np.float32)
    if bf16:
        k, v = synth.bf16_round(k), synth.bf16_round(v)
    dt = torch.bfloat16 if bf16 else torch.float32
    return k, v, torch.from_numpy(k).to(T.DEV).to(dt), torch.from_numpy(v).to(T.DEV).to(dt)


def q_for(batch, hq, d, seed):
    q = synth.bf16_round(np.random.default_rng(seed).standard_normal((batch, hq, d)).astype(np.float32))
    return q, torch.from_numpy(q).to(T.DEV).bfloat16()


def lens_t(lens):
    return torch.as_tensor(np.asarray(lens, np.int32), device=T.DEV)


# (head_dim, hadamard block, group, K bits per head, V bits per head, float16 metadata, bf16 inputs)
FORMATS = [
    (128, 128, 4, [4, 4], [4, 4], False, True),
    (128, 32, 4, [2, 3], [8, 16], False, True),
    (64, 64, 2, [4, 8, 2], [2, 3, 4], False, False),
    (128, 128, 4, [4, 3], [2, 4], True, True),
    (128, 16, 1, [16, 4], [16, 2], False, True),
]


@pytest.mark.parametrize("d,n,g,bk,bv,m16,in_bf16", FORMATS)
def test_fused_append_equals_append_then_decode(d, n, g, bk, bv, m16, in_bf16):
    """Ragged lengths (one sequence empty before the step, one at a page boundary); the new token goes
    to slot lens[b] of each sequence, which the decode then covers (lens + 1)."""
    old = [37, 0, 300, 16, 1000]
    new = [t + 1 for t in old]
    batch, hkv = len(old), len(bk)
    L, lay, cache, ref, table, _, _ = build_case(d, n, g, bk, bv, new, seed=71, chunks=[600, 600],
                                                 meta_fp16=m16)
    kn, vn, knt, vnt = new_rows(batch, hkv, d, 72, in_bf16)
    q, qt = q_for(batch, hkv * g, d, 73)
    start = lens_t(old)
    pool_a, pool_b = cache.pool.clone(), cache.pool.clone()
    seg_a = kvq.Segment(L, pool_a, cache.table, lens_t(new), max(new))
    seg_b = kvq.Segment(L, pool_b, cache.table, lens_t(new), max(new))
    out_a = kvq.kvq_append_decode_attn([seg_a], 0, start, knt, vnt, qt)
    kvq.kvq_quantize_append(L, pool_b, cache.table, start, knt[:, None].contiguous(), vnt[:, None].contiguous())
    out_b = kvq.kvq_decode_attn([seg_b], qt)
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_b), "stored rows differ from kvq_quantize_append's"
    a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
    assert T.max_rel_err(a, b) < SAME
    ref2 = ref.copy()
    O.quantize_append(lay, ref2, table, np.asarray(old), kn[:, None], vn[:, None])
    expect = O.decode_attention([(lay, ref2, table, np.asarray(new))], q.astype(np.float64))
    assert T.max_rel_err(a, expect) <= T.ATTN_TOL


@pytest.mark.parametrize("append_seg", [0, 1])
def test_fused_append_with_a_window_segment(monkeypatch, append_seg):
    """Three segments as at long context: a bf16 window (attended to by the merge kernel), a 4-bit and a
    2-bit segment. The token goes into the window (0) or the 4-bit segment (1); one sequence appends
    nothing (start -1, its lengths unchanged) and one segment is empty for one sequence."""
    monkeypatch.delenv("KVQ_WINDOW_IN_MERGE", raising=False)
    lw, la, lb = [100, 0, 37], [1500, 700, 90], [3000, 16, 0]
    old = [lw, la, lb][append_seg]
    grow = [True, True, False]  # the third sequence appends nothing
    new = [t + 1 if gr else t for t, gr in zip(old, grow)]
    lens = [lw, la, lb]
    full = [list(x) for x in lens]
    full[append_seg] = new
    Lw, layw, cw, rw, tw, _, _ = build_case(128, 32, 4, [16, 16], [16, 16], full[0], seed=81)
    La, laya, ca, ra, ta, _, _ = build_case(128, 32, 4, [4, 4], [4, 4], full[1], seed=82)
    Lb, layb, cb, rb, tb, _, _ = build_case(128, 32, 4, [2, 2], [2, 2], full[2], seed=83)
    caches, lays, refs, tabs, Ls = [cw, ca, cb], [layw, laya, layb], [rw, ra, rb], [tw, ta, tb], [Lw, La, Lb]
    kn, vn, knt, vnt = new_rows(3, 2, 128, 84)
    q, qt = q_for(3, 8, 128, 85)
    start_np = np.asarray([t if gr else -1 for t, gr in zip(old, grow)], np.int32)
    start = torch.as_tensor(start_np, device=T.DEV)

    def segs_over(pools):
        return [kvq.Segment(Ls[i], pools[i], caches[i].table, lens_t(full[i]), max(full[i])) for i in range(3)]

    pools_a = [c.pool.clone() for c in caches]
    pools_b = [c.pool.clone() for c in caches]
    out_a = kvq.kvq_append_decode_attn(segs_over(pools_a), append_seg, start, knt, vnt, qt)
    kvq.kvq_quantize_append(Ls[append_seg], pools_b[append_seg], caches[append_seg].table, start,
                            knt[:, None].contiguous(), vnt[:, None].contiguous())
    out_b = kvq.kvq_decode_attn(segs_over(pools_b), qt)
    torch.cuda.synchronize()
    for pa, pb in zip(pools_a, pools_b):
        assert torch.equal(pa, pb)
    a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
    assert T.max_rel_err(a, b) < SAME
    refs2 = [r.copy() for r in refs]
    keep = np.flatnonzero(start_np >= 0)
    O.quantize_append(lays[append_seg], refs2[append_seg], tabs[append_seg][keep], start_np[keep],
                      kn[keep][:, None], vn[keep][:, None])
    expect = O.decode_attention([(lays[i], refs2[i], tabs[i], np.asarray(full[i])) for i in range(3)],
                                q.astype(np.float64))
    assert T.max_rel_err(a, expect) <= T.ATTN_TOL


def test_fused_append_to_an_unmapped_page_stores_and_attends_nothing():
    """A token whose page has no block is neither stored nor attended to, as with the two calls."""
    old = [40, 47]
    new = [41, 48]
    L, lay, cache, ref, table, _, _ = build_case(128, 128, 4, [4, 4], [2, 2], new, seed=91)
    table2 = table.copy()
    table2[1, 47 // 16] = -1  # the second sequence's last page: unmapped
    tab_t = T.torch_table(table2)
    kn, vn, knt, vnt = new_rows(2, 2, 128, 92)
    q, qt = q_for(2, 8, 128, 93)
    start = lens_t(old)
    pool_a, pool_b = cache.pool.clone(), cache.pool.clone()
    out_a = kvq.kvq_append_decode_attn([kvq.Segment(L, pool_a, tab_t, lens_t(new), 48)], 0, start, knt, vnt, qt)
    kvq.kvq_quantize_append(L, pool_b, tab_t, start, knt[:, None].contiguous(), vnt[:, None].contiguous())
    out_b = kvq.kvq_decode_attn([kvq.Segment(L, pool_b, tab_t, lens_t(new), 48)], qt)
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_b)
    assert torch.equal(pool_a[table[1, 2]], cache.pool[table[1, 2]])  # the unmapped page's block untouched
    assert T.max_rel_err(out_a.cpu().numpy(), out_b.cpu().numpy()) < SAME


@pytest.mark.parametrize("deterministic", [True, False])
def test_fused_step_in_hip_graph_matches_eager(monkeypatch, deterministic):
    """The one-call step captured as a graph over two segments (the partial call forks onto a side stream
    inside the capture), replayed three times with eager work between: every replay equals the eager
    step. The token's slot is rewritten with the same values, so each step sees the same cache."""
    if deterministic:
        monkeypatch.setenv("KVQ_DECODE_DETERMINISTIC", "1")
    lens = [300, 1500]
    new = [t + 1 for t in lens]
    L1, _, c1, _, _, _, _ = build_case(128, 128, 4, [4, 4], [4, 4], lens, seed=61)
    L2, _, c2, _, _, _, _ = build_case(128, 128, 4, [2, 8], [2, 3], new, seed=62)
    segs = [c1.segment(lens), c2.segment(new)]
    _, _, knt, vnt = new_rows(2, 2, 128, 63)
    _, qt = q_for(2, 8, 128, 64)
    start = lens_t(lens)
    ws = kvq.decode_workspace(segs, 2, T.DEV)
    out = torch.empty((2, 8, 128), dtype=torch.float32, device=T.DEV)
    step = kvq.prepare_append_decode_attn(segs, 1, start, knt, vnt, qt, out, ws)
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        out.zero_()
        other = kvq.kvq_decode_attn(segs, qt)  # eager work between replays (the token is in the cache now)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        if deterministic:
            assert torch.equal(out, eager)
        else:
            assert T.rel(out.cpu().numpy(), eager.cpu().numpy()) < 1e-5
        assert T.rel(other.cpu().numpy(), eager.cpu().numpy()) < 1e-5


def test_fused_halves_equal_the_one_call(monkeypatch):
    """kvq_append_decode_partial then kvq_append_decode_merge on one stream is kvq_append_decode_attn (the
    fixed page order: bitwise)."""
    monkeypatch.setenv("KVQ_DECODE_DETERMINISTIC", "1")
    old = [500, 33]
    new = [t + 1 for t in old]
    L, _, cache, _, _, _, _ = build_case(128, 128, 4, [4, 2], [4, 3], new, seed=95)
    _, _, knt, vnt = new_rows(2, 2, 128, 96)
    _, qt = q_for(2, 8, 128, 97)
    start = lens_t(old)
    pool_a, pool_b = cache.pool.clone(), cache.pool.clone()
    seg_a = [kvq.Segment(L, pool_a, cache.table, lens_t(new), max(new))]
    seg_b = [kvq.Segment(L, pool_b, cache.table, lens_t(new), max(new))]
    out_a = kvq.kvq_append_decode_attn(seg_a, 0, start, knt, vnt, qt)
    ws = kvq.decode_workspace(seg_b, 2, T.DEV)
    out_b = torch.empty_like(out_a)
    kvq.prepare_append_decode_partial(seg_b, 0, start, knt, vnt, qt, ws)()
    kvq.prepare_append_decode_merge(seg_b, 0, start, 2, out_b, ws)()
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_b)
    assert torch.equal(out_a, out_b)
