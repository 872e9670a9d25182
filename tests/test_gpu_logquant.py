"""GPU parity of LogQuant's dynamic schedule (LogQuant page, Methodology 2).

A cache of three segments (bf16 window ring, middle precision, low precision)
is prefilled by class, then grown token by token through the C ABI:
kvq_logquant_advance plans each step, kvq_logquant_requant moves the rows
that change class, and kvq_quantize_append writes the new token into the
window. The oracle follows the same tokens on the CPU from the original
inputs: every token starts as the bf16 rotated row, and each class change
re-quantizes the values the token holds (oracle.requantize_row). Compared:
every stored row of every segment (codes bit-exact up to rounding ties,
metadata within a few ulp) and the decode output over the three segments
(max relative error per output vector at most 2e-3).
"""

import numpy as np
import pytest
import torch

from oracle import kvq_oracle as O
from quantized_decode_attention_03_amd import kvq
from tests import kvq_testlib as T

pytestmark = pytest.mark.gpu


class OracleTokens:
    """The oracle's stored representation of every token of one sequence, per (head, half)."""

    def __init__(self, hkv, d, n, bits, m16):
        self.hkv, self.d, self.n, self.bits = hkv, d, n, bits  # bits[cls][half][h]
        self.m16 = m16  # float16 metadata in the middle and low segments
        self.rep = {}  # (pos, h, half) -> (bits, codes, s, mn, values, source values)

    def store(self, pos, cls, x_rows):
        """A token stored straight from its original rows x_rows [2][hkv][d] (prefill or append)."""
        for half in range(2):
            xr = O.rotate(x_rows[half], self.n)
            for h in range(self.hkv):
                b = self.bits[cls][half][h]
                self.rep[(pos, h, half)] = self._encode(xr[h:h + 1], b)

    def move(self, pos, cls):
        """A token re-stored at class cls from the values it holds."""
        for half in range(2):
            for h in range(self.hkv):
                vals = self.rep[(pos, h, half)][4]
                self.rep[(pos, h, half)] = self._encode(vals, self.bits[cls][half][h], requant=True)

    def _encode(self, src, b, requant=False):
        src = np.asarray(src, np.float32)
        if b == 16:
            bits16 = O.float32_to_bf16_bits(src)
            return (16, bits16, None, None, O.bf16_bits_to_float32(bits16), src)
        if requant:
            codes, s, mn = O.requantize_row(src, b, meta_fp16=self.m16)
        else:
            codes, s, mn = O.quantize_rows_fp16_meta(src, b) if self.m16 else O.quantize_rows(src, b)
        return (b, codes, s, mn, O.dequantize_rows(codes, s, mn), src)

    def values(self, positions, h, half):
        return np.concatenate([self.rep[(p, h, half)][4] for p in positions]).astype(np.float64)


def gpu_rows(pool_np, L, table_np, seq, slots, h, half):
    area = (L.k_off if half == 0 else L.v_off)[h]
    bits = (L.bits_k if half == 0 else L.bits_v)[h]
    return T.gather_rows(pool_np, L.block_bytes, table_np, seq, np.asarray(slots), area, L.head_dim, bits,
                         bool(L.meta_fp16))


def oracle_rows(tok, positions, h, half):
    reps = [tok.rep[(p, h, half)] for p in positions]
    b = reps[0][0]
    src = np.concatenate([r[5] for r in reps])
    if b == 16:
        return np.concatenate([r[1] for r in reps]).view(np.uint8).reshape(len(reps), -1), None, src, 16
    rows = O.pack_codes(np.concatenate([r[1] for r in reps]), b)
    meta = np.stack([np.concatenate([r[2] for r in reps]).astype(np.float32),
                     np.concatenate([r[3] for r in reps]).astype(np.float32)], 1)
    return rows, meta, src, b


@pytest.mark.parametrize("d,n,window,starts,steps,mid_bits,low_bits,m16", [
    (64, 64, 16, [300, 77], 150, ([4, 8], [4, 3]), ([2, 2], [2, 3]), False),
    (128, 32, 8, [129, 1], 200, ([4, 4], [4, 4]), ([2, 2], [2, 2]), False),
    (128, 128, 16, [200, 33], 120, ([4, 4], [4, 4]), ([2, 3], [2, 2]), True),
])
def test_logquant_dynamic_steps_match_oracle(d, n, window, starts, steps, mid_bits, low_bits, m16):
    hkv, group, batch = 2, 2, len(starts)
    rng = np.random.default_rng(d + window)
    final = [t + steps for t in starts]
    total_max = max(final)
    x = rng.standard_normal((batch, total_max, 2, hkv, d)).astype(np.float32)
    x[:, :, 0] *= rng.uniform(0.5, 3.0, (1, 1, hkv, d)).astype(np.float32)  # key-like channel scales
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)  # bf16-representable inputs
    q = rng.standard_normal((batch, hkv * group, d)).astype(np.float32)

    L = [kvq.kvq_layout_init(hkv, group, d, n, [16] * hkv, [16] * hkv),
         kvq.kvq_layout_init(hkv, group, d, n, mid_bits[0], mid_bits[1], meta_fp16=m16),
         kvq.kvq_layout_init(hkv, group, d, n, low_bits[0], low_bits[1], meta_fp16=m16)]
    cap = [window, 256, total_max]
    tables, caches = [], []
    for c in range(3):
        n_blocks = batch * (-(-cap[c] // 16)) + 2
        tables.append(T.alloc_tables(batch, [cap[c]] * batch, n_blocks, seed=70 + c))
        caches.append(T.GpuCache(L[c], n_blocks, tables[c]))

    bits = [[[16] * hkv] * 2, [list(mid_bits[0]), list(mid_bits[1])], [list(low_bits[0]), list(low_bits[1])]]
    toks = [OracleTokens(hkv, d, n, bits, m16) for _ in range(batch)]
    st = kvq.LogQuantStates(batch, window, cap_mid=cap[1])
    low_pos = []
    dev = T.DEV

    def to_dev(rows):  # [n_tok, 2, hkv, d] -> k, v [1, n_tok, hkv, d] bf16
        t = torch.from_numpy(np.ascontiguousarray(rows)).to(dev).to(torch.bfloat16)
        return t[None, :, 0].contiguous(), t[None, :, 1].contiguous()

    # ---- prefill by class ----
    for b in range(batch):
        t0 = starts[b]
        cls = kvq.kvq_logquant_dynamic_classes(t0, window).astype(np.int32)
        assert np.array_equal(cls, O.logquant_dynamic_map(t0, window))
        for c in range(3):
            pos = np.flatnonzero(cls == c)
            for p in pos:
                toks[b].store(int(p), c, x[b, p])
            sub = torch.from_numpy(tables[c][b:b + 1].copy()).to(dev)
            if c == 0:
                for p in pos:  # ring slot p mod W
                    k, v = to_dev(x[b, p:p + 1])
                    kvq.kvq_quantize_append(L[0], caches[0].pool, sub,
                                            torch.tensor([p % window], dtype=torch.int32, device=dev), k, v)
            elif len(pos):
                k, v = to_dev(x[b, pos])
                kvq.kvq_quantize_append(L[c], caches[c].pool, sub, torch.zeros(1, dtype=torch.int32, device=dev), k, v)
        st.init(b, t0)
        low_pos.append([int(p) for p in np.flatnonzero(cls == 2)])

    # ---- grow token by token ----
    segs = [caches[c].segment([cap[c]] * batch) for c in range(3)]
    table_dev = caches[0].table
    # the requant is called prepared (arguments marshalled once, moves read at each call) on even
    # steps and directly on odd ones
    requant = kvq.prepare_logquant_requant(segs[0], segs[1], segs[2], batch, st.moves)
    for step in range(steps):
        totals = [int(t) for t in st.field("total")]
        before_mid = [st.mid_pos[b, :st.states[b].n_mid].copy() for b in range(batch)]
        moves = st.advance()
        if step % 2 == 0:
            requant()
        else:
            kvq.kvq_logquant_requant(segs[0], segs[1], segs[2], batch, moves)
        mv = st.move_array()
        new = np.stack([x[b, totals[b]] for b in range(batch)])  # [batch, 2, hkv, d]
        nt = torch.from_numpy(new).to(dev).to(torch.bfloat16)
        kvq.kvq_quantize_append(L[0], caches[0].pool, table_dev, torch.from_numpy(mv[:, 4].astype(np.int32)).to(dev),
                                nt[:, None, 0].contiguous(), nt[:, None, 1].contiguous())
        for b in range(batch):
            for p, a, c in O.logquant_transitions(totals[b], window):
                toks[b].move(p, c)
                if (a, c) == (1, 2):
                    assert before_mid[b][mv[b, 2]] == p and mv[b, 3] == len(low_pos[b])
                    low_pos[b].append(p)
            toks[b].store(totals[b], 0, x[b, totals[b]])
    torch.cuda.synchronize()

    # ---- every stored row against the oracle ----
    stats = T.CodeStats()
    pools = [caches[c].pool.cpu().numpy() for c in range(3)]
    for b in range(batch):
        t = final[b]
        cls = O.logquant_dynamic_map(t, window)
        held = [[p % window for p in range(max(0, t - window), t)], list(range(st.states[b].n_mid)),
                list(range(len(low_pos[b])))]
        positions = [list(range(max(0, t - window), t)), [int(p) for p in st.mid_pos[b, :st.states[b].n_mid]],
                     low_pos[b]]
        for c in range(3):
            assert sorted(positions[c]) == np.flatnonzero(cls == c).tolist()
            if not positions[c]:
                continue
            for h in range(hkv):
                for half in range(2):
                    g, gm = gpu_rows(pools[c], L[c], tables[c], b, held[c], h, half)
                    r, rm, src, bb = oracle_rows(toks[b], positions[c], h, half)
                    T.compare_rows(g, gm, r, rm, src, bb, d, stats, m16 and c > 0)
    assert stats.rate <= 1e-5

    # ---- decode over the three segments ----
    lens = [[min(t, window) for t in final], [int(v) for v in st.field("n_mid")], [len(lp) for lp in low_pos]]
    dsegs = [caches[c].segment(lens[c]) for c in range(3)]
    out = kvq.kvq_decode_attn(dsegs, torch.from_numpy(q).to(dev)).cpu().numpy()
    for b in range(batch):
        allpos = list(range(final[b]))
        qr = O.rotate(q[b], n).astype(np.float64)
        ref = np.zeros((hkv * group, d))
        for g in range(hkv * group):
            h = g // group
            o = O.attention_plain(qr[g], toks[b].values(allpos, h, 0), toks[b].values(allpos, h, 1))
            ref[g] = O.unrotate(o[None], n)[0]
        assert T.max_rel_err(out[b], ref) <= T.ATTN_TOL
