"""Seeded synthetic inputs for the quantized KV-cache workloads.

Random draws and shapes only: nothing in this module rotates, quantizes,
packs, allocates or attends. The same draws feed the HIP library and, in the
tests, the CPU oracle.

Workload shapes (context, batch, heads, head_dim) and value distributions come
from the decode workloads the library is measured on:

* a tiny layer: batch 1, 4 KV heads x 4 query heads, head_dim 64, 1024
  tokens, fp32 K/V ~ N(0, 1) with 2 fixed outlier channels per head scaled
  x20 in K;
* a Llama-3-8B-shaped layer: 8 KV heads x 4 query heads, head_dim 128, bf16,
  K = Z * s_c + mu_c with 4 fixed outlier channels per head (s_c = 15, else 1)
  and per-channel offsets mu_c ~ N(0, 2) (variance 2), V ~ N(0, 1);
* per-head sensitivities lognormal(0, 1) times the U-shaped layer profile
  1 + 3 ((l - 15.5) / 15.5)^2.
"""

import numpy as np

try:  # torch is only needed for the on-device generators
    import torch
except ImportError:  # pragma: no cover - torch is present in every supported setup
    torch = None


# ---------------------------------------------------------------------------
# numpy (host) generators: small cases shared by the oracle tests and parity
# ---------------------------------------------------------------------------

def outlier_channels(rng, hkv, d, count):
    """`count` distinct channels per head, fixed across tokens."""
    return np.stack([rng.choice(d, size=count, replace=False) for _ in range(hkv)])


def tiny_layer(seed=1, batch=1, tokens=1024, hkv=4, group=4, d=64,
               n_outliers=2, outlier_scale=20.0):
    """fp32 K, V [batch, tokens, hkv, d] and q [batch, hkv*group, d]."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((batch, tokens, hkv, d)).astype(np.float32)
    v = rng.standard_normal((batch, tokens, hkv, d)).astype(np.float32)
    ch = outlier_channels(rng, hkv, d, n_outliers)
    for h in range(hkv):
        k[:, :, h, ch[h]] *= np.float32(outlier_scale)
    q = rng.standard_normal((batch, hkv * group, d)).astype(np.float32)
    return k, v, q


def bf16_round(x):
    """Round float32 values to the nearest bfloat16 (half to even), as float32.

    This is the storage type of the inputs, not a step of the method.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def llama_layer_np(seed, batch, tokens, hkv=8, group=4, d=128, n_outliers=4,
                   outlier_scale=15.0, offset_var=2.0):
    """Host version of the Llama-shaped layer; values are bf16-representable fp32."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((batch, tokens, hkv, d)).astype(np.float32)
    scale = np.ones((hkv, d), dtype=np.float32)
    ch = outlier_channels(rng, hkv, d, n_outliers)
    for h in range(hkv):
        scale[h, ch[h]] = outlier_scale
    mu = (rng.standard_normal((hkv, d)) * np.sqrt(offset_var)).astype(np.float32)
    k = bf16_round(z * scale + mu)
    v = bf16_round(rng.standard_normal((batch, tokens, hkv, d)).astype(np.float32))
    q = bf16_round(rng.standard_normal((batch, hkv * group, d)).astype(np.float32))
    return k, v, q


def free_list(n_blocks, seed):
    """A seeded permutation of the block ids [0, n_blocks)."""
    return np.random.default_rng(seed).permutation(n_blocks).astype(np.int32)


def sensitivities(layers, heads, seed):
    """lognormal(0, 1) x (1 + 3 ((l - 15.5) / 15.5)^2), shape [layers, heads]."""
    rng = np.random.default_rng(seed)
    base = rng.lognormal(0.0, 1.0, size=(layers, heads))
    mid = (layers - 1) / 2.0
    prof = 1.0 + 3.0 * ((np.arange(layers) - mid) / mid) ** 2
    return base * prof[:, None]


# ---------------------------------------------------------------------------
# torch (device) generators: full-size workloads
# ---------------------------------------------------------------------------

def llama_layer_torch(seed, batch, tokens, hkv=8, group=4, d=128, n_outliers=4,
                      outlier_scale=15.0, offset_var=2.0, device="cuda"):
    """bf16 K, V [batch, tokens, hkv, d] and q [batch, hkv*group, d] on `device`.

    The outlier channels and offsets are drawn on the host from `seed`; the
    bulk normals are drawn on the device from a generator seeded with `seed`.
    """
    if torch is None:
        raise RuntimeError("torch is required for device inputs")
    rng = np.random.default_rng(seed)
    scale = np.ones((hkv, d), dtype=np.float32)
    ch = outlier_channels(rng, hkv, d, n_outliers)
    for h in range(hkv):
        scale[h, ch[h]] = outlier_scale
    mu = (rng.standard_normal((hkv, d)) * np.sqrt(offset_var)).astype(np.float32)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    scale_t = torch.from_numpy(scale).to(device)
    mu_t = torch.from_numpy(mu).to(device)
    k = torch.empty((batch, tokens, hkv, d), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    # draw in batch slices to bound the fp32 temporaries
    for b in range(batch):
        z = torch.randn((tokens, hkv, d), generator=gen, device=device, dtype=torch.float32)
        k[b] = (z * scale_t + mu_t).to(torch.bfloat16)
        v[b] = torch.randn((tokens, hkv, d), generator=gen, device=device,
                           dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((batch, hkv * group, d), generator=gen, device=device,
                    dtype=torch.float32).to(torch.bfloat16)
    return k, v, q
