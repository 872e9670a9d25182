"""Plain CPU oracle for the quantized KV-cache hot path.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module. The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
imports nothing from the product: the two share no code.

Everything here is the plain definition of what the method computes, written
for a reader to check against the source pages by eye:

* Rotation: block-diagonal Hadamard rotation of each head row, applied as an
  explicit +-1 matrix product in float64, one 1/sqrt(n) scaling, then rounded
  to float32.
  Source: "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World
  LLM Serving" (gist.science/ar/paper/2604.19157), section 2 ("shuffle before
  you shrink": block-diagonal Hadamard rotation spreads outliers).
* Quantization: token-wise asymmetric min/max quantization to b bits in
  float32. Source: SAW-INT4 page, summary and section 2 (token-wise
  quantization after the rotation); RateQuant page (gist.science/ar/paper/
  2605.06675), Methodology stage 3 (per-token asymmetric quantization for the
  values in KIVI).
* Per-head bit widths that differ between K and V: RateQuant page,
  Methodology stage 3 (K/V decoupling into 2N components); "Quantize What
  Counts: More for Keys, Less for Values" page (gist.science/ar/paper/
  2502.15075), section "The solution".
* Paged storage in uniform blocks: SAW-INT4 page, section 1 (PagedAttention
  is built on uniform blocks).
* Attention: softmax(q K^T / sqrt(d)) V over every cached token, with the
  order of tokens irrelevant. Source: LogQuant page (gist.science/ar/paper/
  2503.19950), technical summary, Methodology section 4 (A.V = A_P.V_P).
* Bit allocation: RateQuant page, Methodology stage 1 (D(b) = alpha*beta^-b,
  budgeted objective, reverse water-filling closed form, AM/GM bound) and
  stage 3 (greedy marginal-gain integer allocation).
* Long-context precision map: LogQuant page, technical summary, Methodology
  section 2 (recent window at full precision, then windows of decreasing
  density over growing spans).

Where the pages leave a step open, the reading taken is stated at the
function that implements it.

Every function is pinned by the `not gpu` tests against closed forms,
invariants and brute force; none is marked "parity unpinned".
"""

import math

import numpy as np

BLOCK_TOKENS = 16
META_BYTES = 8  # float32 scale + float32 minimum per (token, head) row


# ---------------------------------------------------------------------------
# Rotation (SAW-INT4 page, section 2)
# ---------------------------------------------------------------------------

def hadamard_pm1(n):
    """Sylvester Hadamard matrix of order n with entries +-1, natural order:
    H[i][j] = (-1)^popcount(i & j)."""
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    idx = np.arange(n)
    parity = np.zeros((n, n), dtype=np.int64)
    both = idx[:, None] & idx[None, :]
    for bit in range(max(1, n.bit_length())):
        parity ^= (both >> bit) & 1
    return np.where(parity == 0, 1.0, -1.0)


def hadamard_matrix(n):
    """Orthonormal Hadamard matrix H_n / sqrt(n) in Sylvester (natural) order.

    The pages say only "block-diagonal Hadamard"; this reading takes the
    Sylvester matrix with no random sign flips, normalised so that H^T H = I.
    """
    return hadamard_pm1(n) / math.sqrt(n)


def rotate(x, n):
    """x' = blockdiag(H_n, ..., H_n) x / sqrt(n) over the last axis, rounded to fp32.

    Blocks are contiguous channel ranges [k*n, (k+1)*n). The +-1 matrix product
    is taken in fp64 (exact for bf16 or fp32 inputs of moderate dynamic range),
    then scaled once by 1/sqrt(n) in fp64, then rounded to fp32: the value of the
    orthonormal rotation up to that last rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % n:
        raise ValueError("head_dim must be a multiple of the Hadamard block")
    h = hadamard_pm1(n)
    blocks = x.reshape(x.shape[:-1] + (d // n, n))
    y = np.matmul(blocks, h.T)  # y_k = H x_k for each block k
    y = y * (1.0 / math.sqrt(n))
    return y.reshape(x.shape).astype(np.float32)


def unrotate(y, n):
    """R^T y over the last axis in fp64 (returns fp64)."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    h = hadamard_pm1(n)
    blocks = y.reshape(y.shape[:-1] + (d // n, n))
    x = np.matmul(blocks, h) * (1.0 / math.sqrt(n))  # x_k = H^T y_k / sqrt(n)
    return x.reshape(y.shape)


# ---------------------------------------------------------------------------
# Token-wise asymmetric quantization (SAW-INT4 page; RateQuant Methodology 3)
# ---------------------------------------------------------------------------

def quantize_rows(xr, b):
    """Quantize each row of float32 `xr` (shape [..., d]) to b-bit codes.

    Per row, all in float32:
      mn = min(x), mx = max(x)
      if mx == mn: s = 0, every code 0 (the dequantized row is mn)
      else: s = (mx - mn) / (2^b - 1), inv = (2^b - 1) / (mx - mn)
      c = clamp(round_half_even((x - mn) * inv), 0, 2^b - 1)
    Returns (codes uint8, s float32, mn float32). The zero point is the row
    minimum itself (a float), not an integer zero point.
    """
    xr = np.asarray(xr, dtype=np.float32)
    qmax = np.float32(2 ** b - 1)
    mn = xr.min(axis=-1)
    mx = xr.max(axis=-1)
    rng = (mx - mn).astype(np.float32)
    nonconst = rng > 0
    safe = np.where(nonconst, rng, np.float32(1))
    s = np.where(nonconst, safe / qmax, np.float32(0)).astype(np.float32)
    inv = np.where(nonconst, qmax / safe, np.float32(0)).astype(np.float32)
    u = ((xr - mn[..., None]).astype(np.float32) * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(u), 0, qmax).astype(np.uint8)
    return codes, s, mn.astype(np.float32)


def float16_down(x):
    """The largest float16 value <= x (float32 input, within the float16 range)."""
    x = np.asarray(x, dtype=np.float32)
    h = x.astype(np.float16)  # round half to even
    with np.errstate(over="ignore"):  # (the unused branch of the largest values)
        return np.where(h.astype(np.float32) > x, np.nextafter(h, np.float16(-np.inf)), h).astype(np.float16)


def float16_up(x):
    """The smallest float16 value >= x."""
    x = np.asarray(x, dtype=np.float32)
    h = x.astype(np.float16)
    with np.errstate(over="ignore"):
        return np.where(h.astype(np.float32) < x, np.nextafter(h, np.float16(np.inf)), h).astype(np.float16)


def quantize_rows_fp16_meta(xr, b):
    """quantize_rows with the scale and minimum stored as float16.

    The float16 pair has to bound the row for the codes to fit: the minimum
    is rounded down, mn = fp16_down(min x), and the scale up,
    s = fp16_up((max x - mn) / (2^b - 1)) (both operations in float32, so the
    bound holds up to their rounding, and the clamp absorbs the rest). Then
    inv = 1 / s and c = clamp(round_half_even((x - mn) * inv), 0, 2^b - 1),
    in float32. A row with max x == mn gets s = 0 and codes 0. Values must lie
    within the float16 range. Returns (codes, s, mn) with s, mn float16.
    """
    xr = np.asarray(xr, dtype=np.float32)
    qmax = np.float32(2 ** b - 1)
    mn = float16_down(xr.min(axis=-1))
    rng = (xr.max(axis=-1) - mn.astype(np.float32)).astype(np.float32)
    nonconst = rng > 0
    s = np.where(nonconst, float16_up((np.where(nonconst, rng, np.float32(1)) / qmax).astype(np.float32)),
                 np.float16(0)).astype(np.float16)
    s32 = s.astype(np.float32)
    inv = np.where(nonconst, np.float32(1) / np.where(nonconst, s32, np.float32(1)), np.float32(0)).astype(np.float32)
    u = ((xr - mn.astype(np.float32)[..., None]).astype(np.float32) * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(u), 0, qmax).astype(np.uint8)
    return codes, s, mn


def quantize_cols(xr, b):
    """Per-channel quantization of one group of rows (xr [tokens, d], float32):
    the KIVI-style key granularity that the RateQuant page names (Methodology 3,
    per-channel symmetric keys in KIVI) and the LogQuant page uses (Methodology
    5, key-per-channel). Here the group is the 16 tokens of a page and the
    scale is asymmetric, as for rows: per channel c over the group's tokens,
    mn_c = min, mx_c = max, s_c = (mx_c - mn_c) / (2^b - 1),
    inv_c = (2^b - 1) / (mx_c - mn_c), code = clamp(rne((x - mn_c) * inv_c)),
    all in float32; a constant channel gets s_c = 0 and codes 0.
    Returns (codes [tokens, d] uint8, s [d], mn [d]).
    """
    xr = np.asarray(xr, dtype=np.float32)
    qmax = np.float32(2 ** b - 1)
    mn = xr.min(axis=0)
    rng = (xr.max(axis=0) - mn).astype(np.float32)
    nonconst = rng > 0
    safe = np.where(nonconst, rng, np.float32(1))
    s = np.where(nonconst, safe / qmax, np.float32(0)).astype(np.float32)
    inv = np.where(nonconst, qmax / safe, np.float32(0)).astype(np.float32)
    u = ((xr - mn[None, :]).astype(np.float32) * inv[None, :]).astype(np.float32)
    return np.clip(np.rint(u), 0, qmax).astype(np.uint8), s, mn.astype(np.float32)


def dequantize_rows(codes, s, mn):
    """x_hat = c * s + mn in float32 (a rounded product, then a rounded sum);
    float16 metadata is widened to float32 (exactly) first."""
    s = np.asarray(s).astype(np.float32)
    mn = np.asarray(mn).astype(np.float32)
    prod = (codes.astype(np.float32) * s[..., None]).astype(np.float32)
    return (prod + mn[..., None]).astype(np.float32)


def float32_to_bf16_bits(x):
    """Round float32 to bfloat16 (round half to even); returns uint16 bits."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_float32(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# Bit packing
# ---------------------------------------------------------------------------

def pack_codes(codes, b):
    """Dense little-endian bit-stream per row.

    Code j occupies bits [j*b, j*b + b) of the row's stream; stream bit i sits
    in byte i // 8 at bit position i % 8 (so 32-bit words are little-endian).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    d = codes.shape[-1]
    if (d * b) % 8:
        raise ValueError("row does not fill whole bytes")
    bits = (codes[..., :, None] >> np.arange(b, dtype=np.uint8)) & 1
    bits = bits.reshape(codes.shape[:-1] + (d * b,))
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_codes(packed, b, d):
    packed = np.asarray(packed, dtype=np.uint8)
    bits = np.unpackbits(packed, axis=-1, bitorder="little")[..., : d * b]
    bits = bits.reshape(packed.shape[:-1] + (d, b)).astype(np.uint16)
    weights = (1 << np.arange(b, dtype=np.uint16))
    return (bits * weights).sum(axis=-1).astype(np.uint8)


# ---------------------------------------------------------------------------
# Paged block layout (SAW-INT4 page, section 1: uniform blocks)
# ---------------------------------------------------------------------------

def row_bytes(d, b):
    """Bytes of one stored row: packed codes (b in {2,3,4,8}) or bf16 (b = 16)."""
    return d * b // 8


def segment_bytes(d, b, meta_bytes=META_BYTES):
    """One head's K (or V) area in a block: 16 rows, then 16 metadata pairs
    (meta_bytes each: 8 for a float32 pair, 4 for a float16 pair).

    b = 16 rows are stored as bf16 of the rotated row and carry no metadata.
    """
    meta = 0 if b == 16 else BLOCK_TOKENS * meta_bytes
    return BLOCK_TOKENS * row_bytes(d, b) + meta


def key_area_bytes(d, b, meta_bytes=META_BYTES, key_per_channel=False):
    """A head's K area: per-token metadata as segment_bytes, or with per-channel
    keys 16 code rows then one float32 {s, mn} pair per channel (d pairs)."""
    if key_per_channel and b != 16:
        return BLOCK_TOKENS * row_bytes(d, b) + d * META_BYTES
    return segment_bytes(d, b, meta_bytes)


def block_layout(num_kv_heads, d, bits_k, bits_v, meta_bytes=META_BYTES, key_per_channel=False):
    """Byte offsets of every head's K and V area inside a block.

    Order: K head 0, K head 1, ..., then V head 0, V head 1, ...
    Returns (k_off list, v_off list, block_bytes).
    """
    off = 0
    k_off, v_off = [], []
    for h in range(num_kv_heads):
        k_off.append(off)
        off += key_area_bytes(d, bits_k[h], meta_bytes, key_per_channel)
    for h in range(num_kv_heads):
        v_off.append(off)
        off += segment_bytes(d, bits_v[h], meta_bytes)
    return k_off, v_off, off


class Layout:
    """The cache geometry of one pool: heads, head_dim, Hadamard block, bits."""

    def __init__(self, num_kv_heads, group, head_dim, had_block, bits_k, bits_v, meta_fp16=False,
                 key_per_channel=False):
        self.meta_fp16 = bool(meta_fp16)
        self.key_per_channel = bool(key_per_channel)
        if self.meta_fp16 and self.key_per_channel:
            raise ValueError("per-channel keys keep float32 metadata")
        self.meta_bytes = 4 if self.meta_fp16 else META_BYTES
        self.hkv = int(num_kv_heads)
        self.group = int(group)
        self.d = int(head_dim)
        self.n = int(had_block)
        self.bits_k = [int(b) for b in bits_k]
        self.bits_v = [int(b) for b in bits_v]
        self.k_off, self.v_off, self.block_bytes = block_layout(
            self.hkv, self.d, self.bits_k, self.bits_v, self.meta_bytes, self.key_per_channel)


# ---------------------------------------------------------------------------
# Page allocation
# ---------------------------------------------------------------------------

def page_alloc(free_list, cursor, old_len, new_len, table):
    """Give each sequence the blocks it needs to grow from old_len to new_len.

    Blocks are popped from `free_list` front to back, sequence by sequence
    (ascending), and within a sequence by ascending logical block index.
    `table` is [batch, max_blocks] int32 and is updated in place.
    Returns the new cursor. Raises if the free list runs out.
    """
    for seq in range(len(old_len)):
        have = -(-int(old_len[seq]) // BLOCK_TOKENS)
        need = -(-int(new_len[seq]) // BLOCK_TOKENS)
        for lb in range(have, need):
            if cursor >= len(free_list):
                raise RuntimeError("free list exhausted")
            table[seq, lb] = free_list[cursor]
            cursor += 1
    return cursor


# ---------------------------------------------------------------------------
# Quantize-on-append into the paged pool
# ---------------------------------------------------------------------------

def encode_rows(x, n, b, meta_fp16=False):
    """Rotate then quantize rows of x ([..., d]); returns (row bytes, s, mn).

    For b = 16 the stored row is the rotated row rounded to bf16 and s, mn are
    None. With meta_fp16 the float16-metadata quantizer is used.
    """
    xr = rotate(x, n)
    if b == 16:
        return float32_to_bf16_bits(xr).view(np.uint8).reshape(xr.shape[:-1] + (-1,)), None, None
    codes, s, mn = quantize_rows_fp16_meta(xr, b) if meta_fp16 else quantize_rows(xr, b)
    return pack_codes(codes, b), s, mn


def quantize_append(layout, pool, table, start_pos, k, v):
    """Write new K/V rows ([B, n_new, Hkv, d]) at positions start_pos[b] + i.

    pool is uint8 [n_blocks, block_bytes]; table is int32 [B, max_blocks].
    """
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    batch, n_new, hkv, d = k.shape
    if layout.key_per_channel:
        _append_keys_per_channel(layout, pool, table, start_pos, k)
    for which, x, bits, offs in (("k", k, layout.bits_k, layout.k_off),
                                 ("v", v, layout.bits_v, layout.v_off)):
        for h in range(hkv):
            b = bits[h]
            if which == "k" and layout.key_per_channel and b != 16:
                continue  # written per page above
            rb = row_bytes(d, b)
            rows, s, mn = encode_rows(x[:, :, h, :], layout.n, b, layout.meta_fp16)
            for seq in range(batch):
                for i in range(n_new):
                    pos = int(start_pos[seq]) + i
                    blk = int(table[seq, pos // BLOCK_TOKENS])
                    slot = pos % BLOCK_TOKENS
                    base = offs[h]
                    pool[blk, base + slot * rb: base + (slot + 1) * rb] = rows[seq, i]
                    if b != 16:
                        mb = layout.meta_bytes
                        mbase = base + BLOCK_TOKENS * rb + slot * mb
                        meta = np.array([s[seq, i], mn[seq, i]], dtype=np.float16 if layout.meta_fp16 else np.float32)
                        pool[blk, mbase: mbase + mb] = meta.view(np.uint8)


def _append_keys_per_channel(layout, pool, table, start_pos, k):
    """Per-channel keys: each page of 16 new tokens is one quantization group,
    so appends must cover whole pages (start and count multiples of 16)."""
    batch, n_new, hkv, d = k.shape
    if n_new % BLOCK_TOKENS:
        raise ValueError("per-channel keys are appended in whole pages")
    for h in range(hkv):
        b = layout.bits_k[h]
        if b == 16:
            continue
        rb = row_bytes(d, b)
        base = layout.k_off[h]
        xr = rotate(k[:, :, h, :], layout.n)
        for seq in range(batch):
            if int(start_pos[seq]) % BLOCK_TOKENS:
                raise ValueError("per-channel keys are appended in whole pages")
            for i0 in range(0, n_new, BLOCK_TOKENS):
                codes, s, mn = quantize_cols(xr[seq, i0:i0 + BLOCK_TOKENS], b)
                blk = int(table[seq, (int(start_pos[seq]) + i0) // BLOCK_TOKENS])
                pool[blk, base: base + BLOCK_TOKENS * rb] = pack_codes(codes, b).reshape(-1)
                meta = np.stack([s, mn], axis=1).astype(np.float32)  # [d][{s, mn}]
                pool[blk, base + BLOCK_TOKENS * rb: base + BLOCK_TOKENS * rb + d * META_BYTES] = meta.view(np.uint8).reshape(-1)


def read_rows(layout, pool, table_row, pos0, n, h, which):
    """Return the rotated, dequantized fp32 rows [n, d] of one head (K or V)."""
    d = layout.d
    bits = layout.bits_k[h] if which == "k" else layout.bits_v[h]
    base = layout.k_off[h] if which == "k" else layout.v_off[h]
    rb = row_bytes(d, bits)
    pos = pos0 + np.arange(n)
    blk = np.asarray(table_row)[pos // BLOCK_TOKENS].astype(np.int64)
    slot = pos % BLOCK_TOKENS
    cols = base + slot[:, None] * rb + np.arange(rb)[None, :]
    raw = pool[blk[:, None], cols]
    if bits == 16:
        return bf16_bits_to_float32(raw.view(np.uint16).reshape(n, d))
    codes = unpack_codes(raw, bits, d)
    if which == "k" and layout.key_per_channel:
        mcols = base + BLOCK_TOKENS * rb + np.arange(d * META_BYTES)
        meta = pool[blk[:, None], mcols[None, :]].copy().view(np.float32).reshape(n, d, 2)
        prod = (codes.astype(np.float32) * meta[:, :, 0]).astype(np.float32)
        return (prod + meta[:, :, 1]).astype(np.float32)
    mb = layout.meta_bytes
    mcols = base + BLOCK_TOKENS * rb + slot[:, None] * mb + np.arange(mb)[None, :]
    meta = pool[blk[:, None], mcols].copy().view(np.float16 if layout.meta_fp16 else np.float32)
    meta = meta.astype(np.float32).reshape(n, 2)
    return dequantize_rows(codes, meta[:, 0], meta[:, 1])


def dequant(layout, pool, table_row, pos0, n, rotated):
    """K and V rows [n, Hkv, d] of one sequence in float32.

    rotated=True returns the stored (rotated) basis; otherwise R^T x_hat' is
    returned, rounded to float32.
    """
    out_k = np.zeros((n, layout.hkv, layout.d), dtype=np.float32)
    out_v = np.zeros_like(out_k)
    for h in range(layout.hkv):
        for which, out in (("k", out_k), ("v", out_v)):
            rows = read_rows(layout, pool, table_row, pos0, n, h, which)
            out[:, h, :] = rows if rotated else unrotate(rows, layout.n).astype(np.float32)
    return out_k, out_v


# ---------------------------------------------------------------------------
# Decode attention over one or more segments (LogQuant Methodology section 4)
# ---------------------------------------------------------------------------

def decode_attention(segments, q):
    """softmax(q K^T / sqrt(d)) V for one decode query per q-head.

    segments: list of (layout, pool, table [B, max_blocks], seq_lens [B]);
    every segment shares num_kv_heads, group, head_dim and had_block. q is
    [B, Hq, d]. The attended set is the union of every segment's tokens; the
    order of tokens does not change the result.

    Steps: q' = R q (fp64); for KV head h = g // G, z_t = q' . k_hat'_t / sqrt(d)
    over all cached tokens; p = softmax(z) in fp64; o' = sum_t p_t v_hat'_t;
    o = R^T o'. Output float32 [B, Hq, d].
    """
    q = np.asarray(q, dtype=np.float64)
    batch, hq, d = q.shape
    lay0 = segments[0][0]
    g_size, n = lay0.group, lay0.n
    out = np.zeros((batch, hq, d), dtype=np.float32)
    hmat = hadamard_matrix(n)
    for bi in range(batch):
        for h in range(lay0.hkv):
            ks, vs = [], []
            for lay, pool, table, seq_lens in segments:
                t = int(seq_lens[bi])
                if t == 0:
                    continue
                ks.append(read_rows(lay, pool, table[bi], 0, t, h, "k"))
                vs.append(read_rows(lay, pool, table[bi], 0, t, h, "v"))
            if not ks:
                continue  # no tokens: the output stays zero
            kk = np.concatenate(ks).astype(np.float64)
            vv = np.concatenate(vs).astype(np.float64)
            for g in range(h * g_size, (h + 1) * g_size):
                qr = (q[bi, g].reshape(d // n, n) @ hmat.T).reshape(d)
                z = kk @ qr / math.sqrt(d)
                z -= z.max()
                p = np.exp(z)
                p /= p.sum()
                o_rot = p @ vv
                out[bi, g] = unrotate(o_rot, n).astype(np.float32)
    return out


def attention_plain(q, k, v):
    """softmax(q k^T / sqrt(d)) v for one query vector in fp64 (no cache)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = k @ q / math.sqrt(q.shape[-1])
    z -= z.max()
    p = np.exp(z)
    p /= p.sum()
    return p @ v


# ---------------------------------------------------------------------------
# Bit allocation (RateQuant page, Methodology stages 1 and 3)
# ---------------------------------------------------------------------------

def distortion(b, alpha, beta):
    """D(b) = alpha * beta^(-b)."""
    return alpha * beta ** (-np.asarray(b, dtype=np.float64))


def plan_bits_greedy(w, alpha, beta, ladder, budget):
    """Greedy marginal-gain integer allocation of `budget` bits over N heads.

    Every head starts at the smallest ladder width. Each round gives one more
    ladder step to the head whose step has the largest weighted distortion drop
    per bit spent, w_i (D(b) - D(b+)) / (b+ - b), among steps that still fit the
    remaining budget; ties go to the lowest head index. It stops when the budget
    is spent or no step fits. The "per bit" normalisation is this reading of the
    page's "largest drop" for ladders with unequal steps (4 -> 8 costs 4 bits);
    for unit steps the two agree.

    Returns (bits list, leftover bits).
    """
    ladder = sorted(int(b) for b in ladder)
    w = [float(x) for x in w]
    level = [0] * len(w)
    remaining = int(budget) - len(w) * ladder[0]
    if remaining < 0:
        raise ValueError("budget below the smallest allocation")
    while remaining > 0:
        best, best_gain = -1, -1.0
        for i, wi in enumerate(w):
            if level[i] + 1 >= len(ladder):
                continue
            b0, b1 = ladder[level[i]], ladder[level[i] + 1]
            if b1 - b0 > remaining:
                continue
            gain = wi * (alpha * beta ** (-b0) - alpha * beta ** (-b1)) / (b1 - b0)
            if gain > best_gain:
                best, best_gain = i, gain
        if best < 0:
            break
        remaining -= ladder[level[best] + 1] - ladder[level[best]]
        level[best] += 1
    return [ladder[lv] for lv in level], remaining


def plan_bits_greedy_components(w, alpha, beta, ladder, budget):
    """plan_bits_greedy over components that each have their own distortion
    curve D_i(b) = alpha_i * beta_i^(-b).

    RateQuant page, Methodology stage 3 ("K/V decoupling"): the keys and the
    values of every head are separate components (2N of them), each with its
    own fitted curve, and one budget is shared by all of them, so the split
    between keys and values is decided by the allocation itself (the page's
    key result finds 2.85 bits for keys and 2.15 for values at 2.5 on
    average). The rounds are those of plan_bits_greedy: every component
    starts at the smallest ladder width, and each round gives one more ladder
    step to the component with the largest drop per bit,
    w_i (D_i(b) - D_i(b+)) / (b+ - b), among steps that fit the remaining
    budget; ties go to the lowest index; it stops when the budget is spent or
    no step fits. alpha and beta are sequences with one value per component.

    Returns (bits list, leftover bits).
    """
    ladder = sorted(int(b) for b in ladder)
    w = [float(x) for x in w]
    alpha = [float(a) for a in alpha]
    beta = [float(b) for b in beta]
    if not len(w) == len(alpha) == len(beta):
        raise ValueError("one alpha and one beta per component")
    level = [0] * len(w)
    remaining = int(budget) - len(w) * ladder[0]
    if remaining < 0:
        raise ValueError("budget below the smallest allocation")
    while remaining > 0:
        best, best_gain = -1, -1.0
        for i, wi in enumerate(w):
            if level[i] + 1 >= len(ladder):
                continue
            b0, b1 = ladder[level[i]], ladder[level[i] + 1]
            if b1 - b0 > remaining:
                continue
            gain = wi * (alpha[i] * beta[i] ** (-b0) - alpha[i] * beta[i] ** (-b1)) / (b1 - b0)
            if gain > best_gain:
                best, best_gain = i, gain
        if best < 0:
            break
        remaining -= ladder[level[best] + 1] - ladder[level[best]]
        level[best] += 1
    return [ladder[lv] for lv in level], remaining


def waterfill_bits_components(w, alpha, beta, total):
    """Continuous optimum of sum_i w_i alpha_i beta_i^(-b_i) subject to
    sum_i b_i = total, for components with their own curves (the relaxation
    of plan_bits_greedy_components).

    Setting the derivative of the Lagrangian to zero gives
    w_i alpha_i ln(beta_i) beta_i^(-b_i) = lam for every i, so
    b_i = (ln(w_i alpha_i ln beta_i) - ln lam) / ln beta_i, and the budget fixes
    ln lam = (sum_i ln(w_i alpha_i ln beta_i) / ln beta_i - total) /
    sum_i (1 / ln beta_i). With every alpha_i and beta_i equal this is the
    reverse water-filling of waterfill_bits.
    """
    w = np.asarray(w, dtype=np.float64)
    lb = np.log(np.asarray(beta, dtype=np.float64))
    c = np.log(w * np.asarray(alpha, dtype=np.float64) * lb)
    ln_lam = ((c / lb).sum() - float(total)) / (1.0 / lb).sum()
    return (c - ln_lam) / lb


def waterfill_bits(w, beta, b_mean):
    """Continuous optimum b*_i = b_mean + (ln w_i - ln w_bar) / ln beta, w_bar the
    geometric mean of the sensitivities (reverse water-filling)."""
    lw = np.log(np.asarray(w, dtype=np.float64))
    return b_mean + (lw - lw.mean()) / math.log(beta)


def amgm_ratio(w):
    """Arithmetic over geometric mean of the sensitivities."""
    w = np.asarray(w, dtype=np.float64)
    return w.mean() / math.exp(np.log(w).mean())


def quant_mse(x, n, widths):
    """Mean squared quantization error of this quantizer at each width.

    RateQuant page, Methodology 3 ("distortion calibration": the distortion
    curve alpha * beta^-b is fitted per quantizer from measured errors) and
    the pipeline's step 2 (errors at five widths). The quantizer is the one
    this cache stores: each row of x ([..., d]) is rotated (rotate), quantized
    token-wise (quantize_rows) and dequantized (dequantize_rows), all in
    float32; the error of each element against the rotated value is taken in
    float64 (exact for two float32 values), squared, and averaged over every
    element. Returns one float per width.
    """
    xr = rotate(np.asarray(x, dtype=np.float32), n)
    ref = xr.astype(np.float64)
    out = []
    for b in widths:
        codes, s, mn = quantize_rows(xr, b)
        err = dequantize_rows(codes, s, mn).astype(np.float64) - ref
        out.append(float((err * err).sum() / err.size))
    return out


def fit_distortion(bits, mse):
    """Least-squares fit of ln MSE = ln alpha - b ln beta; returns (alpha, beta, r2)."""
    b = np.asarray(bits, dtype=np.float64)
    y = np.log(np.asarray(mse, dtype=np.float64))
    a_mat = np.stack([np.ones_like(b), -b], axis=1)
    coef, *_ = np.linalg.lstsq(a_mat, y, rcond=None)
    pred = a_mat @ coef
    ss_res = float(((y - pred) ** 2).sum())
    ss_tot = float(((y - y.mean()) ** 2).sum())
    return math.exp(coef[0]), math.exp(coef[1]), 1.0 - ss_res / ss_tot


# ---------------------------------------------------------------------------
# Long-context precision map (LogQuant technical summary, Methodology 2)
# ---------------------------------------------------------------------------

def logquant_precision_map(total, window):
    """Precision class of each of `total` tokens (position 0 = oldest).

    0 = the most recent `window` tokens, kept in bf16;
    1 = the log-spaced subset kept at the middle precision;
    2 = everything else, at the lowest precision.
    Let r be the distance behind the window (r = 0 is the newest token outside
    it). Span k covers r in [(2^k - 1) W, (2^(k+1) - 1) W) and keeps every
    2^k-th token of the span, counted from the span's start. This reading
    takes W as both the window and the first span length, which is the choice
    under which the spans tile a 2^m-token context exactly.
    """
    cls = np.full(total, 2, dtype=np.int32)
    for pos in range(total):
        dist = total - 1 - pos  # 0 for the newest token
        if dist < window:
            cls[pos] = 0
            continue
        r = dist - window
        k = 0
        while r >= ((1 << (k + 1)) - 1) * window:
            k += 1
        start = ((1 << k) - 1) * window
        if (r - start) % (1 << k) == 0:
            cls[pos] = 1
    return cls


def logquant_dynamic_map(total, window):
    """Precision class of each of `total` tokens when the cache grows one token
    at a time (LogQuant technical summary, Methodology 2, "dynamic adjustment":
    as tokens arrive, the older windows are thinned by half, keeping tokens at
    regular intervals, so a kept token only ever loses precision).

    Same window and spans as logquant_precision_map. In span k a token at
    position p is kept (class 1) when (p + 1) is a multiple of 2^k: every
    2^k-th token, counted on absolute positions. As the context grows a token
    moves into older spans, where the condition only gets stricter, so its
    class never returns to a higher precision. Span k (2^k W tokens) still
    keeps W of them. When `total` is a multiple of 2^K, K the oldest span
    present, this picks the same tokens as logquant_precision_map (there p is
    kept when p = total - 1 modulo 2^k, which is -1 modulo 2^k).
    """
    cls = np.full(total, 2, dtype=np.int32)
    for pos in range(total):
        dist = total - 1 - pos
        if dist < window:
            cls[pos] = 0
            continue
        r = dist - window
        k = 0
        while r >= ((1 << (k + 1)) - 1) * window:
            k += 1
        if (pos + 1) % (1 << k) == 0:
            cls[pos] = 1
    return cls


def logquant_transitions(total, window):
    """Class changes when token `total` is appended to a cache of `total`
    tokens: [(position, old class, new class)] over the existing positions,
    read off the two dynamic maps (the new token itself enters class 0)."""
    before = logquant_dynamic_map(total, window)
    after = logquant_dynamic_map(total + 1, window)[:total]
    changed = np.flatnonzero(before != after)
    return [(int(p), int(before[p]), int(after[p])) for p in changed]


def requantize_row(x_hat, b, meta_fp16=False):
    """Re-encode a stored row at b bits (LogQuant Methodology 2: a token that
    leaves the window, or the kept subset, is stored again at the lower
    precision). The source is what the cache holds, already in the rotated
    basis: the bf16 window row, or the dequantized middle-precision row. It is
    quantized token-wise exactly like a new row (quantize_rows, or
    quantize_rows_fp16_meta for a destination with float16 metadata)."""
    x_hat = np.asarray(x_hat, dtype=np.float32)
    return quantize_rows_fp16_meta(x_hat, b) if meta_fp16 else quantize_rows(x_hat, b)
