"""Seeded generators for attention inputs with block-structured score mass.

Every generator uses numpy's PCG64 streams and draws in a fixed order, so a
seed names one exact tensor set: shared draws (the centroids) come from
``default_rng(seed)``, and each (batch, head) unit draws from its own stream
``default_rng([seed, b, h])``, which lets units be generated in parallel
threads without changing any value.  Values are drawn in fp32 and,
for bf16 workloads, rounded once to bf16 with round-to-nearest-even (torch's
CPU cast).  Whatever consumes the tensors (the fp64 oracle, the GPU kernels)
reads back exactly those rounded values.

Three families:

* ``clustered_*`` -- keys sit near unit-norm centroids, one centroid per
  128-key tile, so a query near a few centroids scores high on a few tiles and
  low on the rest: the regime in which whole key tiles carry negligible
  softmax mass.
* ``video_dit_field`` -- queries and keys sampled from spatially smooth 3-D
  fields over a (frames, height, width) latent grid plus a bounded locality
  term, so nearby tokens score high: a stand-in for video diffusion
  transformer self-attention.
* ``gumbel_decode`` -- every head of a KV group shares one query direction
  ``u`` and each key's component along ``u`` is chosen so that the scaled
  score ``scale * q.k`` is an independent standard Gumbel draw: a control
  workload whose score statistics are known in closed form at any length.
"""

from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

TILE = 128  # keys per tile that a centroid is assigned to


def _unit_rng(seed: int, *unit: int) -> np.random.Generator:
    return np.random.default_rng([seed, *unit])


def _for_units(units, fn) -> None:
    """Run fn(unit) over all units on a small thread pool (numpy and torch
    release the GIL in the bulk fills and casts)."""
    units = list(units)
    n = min(len(units), max(1, min(16, os.cpu_count() or 1)))
    if n <= 1:
        for u in units:
            fn(u)
        return
    with cf.ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(fn, units))


def bf16_round(x: np.ndarray) -> torch.Tensor:
    """fp32 array -> contiguous bf16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def _to_tensor(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def _torch_dtype(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def _centroids(rng: np.random.Generator, n_c: int, d: int) -> np.ndarray:
    c = rng.standard_normal((n_c, d), dtype=np.float32)
    c /= np.linalg.norm(c, axis=1, keepdims=True)
    return c


def clustered_prefill(seed: int, B: int, Hq: int, Hkv: int, Lq: int, Lk: int, D: int,
                      Dv: int, n_c: int, r: float, query_mode: str, dtype: str = "bf16",
                      sigma: float = 0.5) -> dict:
    """Tile-clustered Q/K/V for a prefill call.

    Draw order: centroids ``C`` (n_c x D, row-normalised) from the shared
    stream; then, from the stream of each (b, kv head): tile centroids ``z``
    (one per 128-key tile), key noise, query centroid choices
    (``query_mode == "row"`` only), query noise for the ``Hq/Hkv`` heads of
    the group, then V ~ N(0, 1).

    ``k = r*C[z_tile] + sigma*eps``.  Queries:

    * ``"row"``: every query row of every head picks its own centroid
      uniformly, ``q = r*C[zq] + sigma*eps``;
    * ``"tile"``: self-attention layout -- query position ``p`` uses the
      centroid of the key tile holding key position ``p + Lk - Lq`` (clamped
      to the key range), with independent noise per head.
    """
    rng = np.random.default_rng(seed)
    g = Hq // Hkv
    nK = -(-Lk // TILE)
    C = _centroids(rng, n_c, D)
    tdt = _torch_dtype(dtype)
    q = torch.empty((B, Hq, Lq, D), dtype=tdt)
    k = torch.empty((B, Hkv, Lk, D), dtype=tdt)
    v = torch.empty((B, Hkv, Lk, Dv), dtype=tdt)
    key_tile_of_query = np.clip(np.arange(Lq) + (Lk - Lq), 0, Lk - 1) // TILE

    def unit(bh):
        b, hk = bh
        rng = _unit_rng(seed, b, hk)
        z = rng.integers(0, n_c, size=nK)
        kz = np.repeat(z, TILE)[:Lk]
        kk = r * C[kz] + sigma * rng.standard_normal((Lk, D), dtype=np.float32)
        if query_mode == "row":
            zq = rng.integers(0, n_c, size=(g, Lq))
        elif query_mode == "tile":
            zq = np.broadcast_to(z[key_tile_of_query], (g, Lq))
        else:
            raise ValueError(f"unknown query_mode {query_mode!r}")
        qq = r * C[zq] + sigma * rng.standard_normal((g, Lq, D), dtype=np.float32)
        vv = rng.standard_normal((Lk, Dv), dtype=np.float32)
        k[b, hk] = _to_tensor(kk, dtype)
        q[b, hk * g:(hk + 1) * g] = _to_tensor(qq, dtype)
        v[b, hk] = _to_tensor(vv, dtype)

    _for_units([(b, hk) for b in range(B) for hk in range(Hkv)], unit)
    return {"q": q, "k": k, "v": v}


def clustered_decode(seed: int, B: int, Hq: int, Hkv: int, Lk: int, D: int, Dv: int,
                     n_c: int, r: float, latent: bool = False, dtype: str = "bf16",
                     sigma: float = 0.5, max_hot: int = 3) -> dict:
    """Tile-clustered single-token decode inputs.

    Draw order: centroids from the shared stream; then, from the stream of
    each (b, kv head): tile centroids, key noise, the token's hot-centroid
    count ``m ~ U{1..max_hot}`` and its ``m`` distinct centroids, query noise for the group's heads, then V (skipped
    when ``latent``: the value rows are then the first ``Dv`` columns of each
    key row, which the consumer reads out of ``k`` itself).

    Every head of a group shares the token's direction
    ``u = normalize(sum of its hot centroids)``: ``q_h = r*u + sigma*eps_h``.
    """
    rng = np.random.default_rng(seed)
    g = Hq // Hkv
    nK = -(-Lk // TILE)
    C = _centroids(rng, n_c, D)
    tdt = _torch_dtype(dtype)
    q = torch.empty((B, Hq, D), dtype=tdt)
    k = torch.empty((B, Hkv, Lk, D), dtype=tdt)
    v = None if latent else torch.empty((B, Hkv, Lk, Dv), dtype=tdt)

    def unit(bh):
        b, hk = bh
        rng = _unit_rng(seed, b, hk)
        z = rng.integers(0, n_c, size=nK)
        kz = np.repeat(z, TILE)[:Lk]
        kk = r * C[kz] + sigma * rng.standard_normal((Lk, D), dtype=np.float32)
        m = int(rng.integers(1, max_hot + 1))
        hot = rng.choice(n_c, size=m, replace=False)
        u = C[hot].sum(axis=0)
        u /= np.linalg.norm(u)
        qq = r * u[None, :] + sigma * rng.standard_normal((g, D), dtype=np.float32)
        k[b, hk] = _to_tensor(kk, dtype)
        q[b, hk * g:(hk + 1) * g] = _to_tensor(qq, dtype)
        if not latent:
            v[b, hk] = _to_tensor(rng.standard_normal((Lk, Dv), dtype=np.float32), dtype)

    _for_units([(b, hk) for b in range(B) for hk in range(Hkv)], unit)
    return {"q": q, "k": k, "v": v}


def video_dit_field(seed: int, B: int, H: int, grid: tuple = (13, 42, 60), n_field: int = 122,
                    alpha: float = 4.0, blur: float = 2.0, noise: float = 0.5,
                    dtype: str = "bf16", heads: int | None = None) -> dict:
    """Smooth-field self-attention inputs over a (T, H, W) latent grid.

    Tokens are flattened frame-major, then row, then column.  Per (b, head):
    ``n_field`` channels, each an N(0,1) grid blurred by a Gaussian of ``blur``
    voxels (reflecting borders) and standardised per channel, give the field
    ``F``; ``q = F + noise*eps``, ``k = F + noise*eps'``.  Six locality
    channels ``alpha*[cos(pi*p_a/N_a), sin(pi*p_a/N_a)]`` for each grid axis
    ``a`` are appended identically to q and k; their dot product is
    ``alpha^2 * sum_a cos(pi*(p_a - p'_a)/N_a)``, largest for nearby tokens
    and bounded, so bf16 holds it.  V ~ N(0, 1).  Draw order, from the
    stream of each (b, head): field grids, query noise, key noise, V.

    ``heads`` generates only the first ``heads`` heads (a bounded sample of
    the full tensor, bit-identical to its leading heads).
    """
    from scipy.ndimage import gaussian_filter

    T, Hh, W = grid
    L = T * Hh * W
    D = n_field + 6
    nh = H if heads is None else heads
    pt, ph, pw = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
    loc = []
    for p, n in ((pt, T), (ph, Hh), (pw, W)):
        ang = np.pi * p.reshape(-1).astype(np.float64) / n
        loc += [np.cos(ang), np.sin(ang)]
    loc = (alpha * np.stack(loc, axis=1)).astype(np.float32)  # [L, 6]
    tdt = _torch_dtype(dtype)
    q = torch.empty((B, nh, L, D), dtype=tdt)
    k = torch.empty((B, nh, L, D), dtype=tdt)
    v = torch.empty((B, nh, L, D), dtype=tdt)
    def unit(bh):
        b, h = bh
        rng = _unit_rng(seed, b, h)
        f = rng.standard_normal((n_field, T, Hh, W), dtype=np.float32)
        f = gaussian_filter(f, sigma=(0, blur, blur, blur), mode="reflect")
        f = f.reshape(n_field, L)
        f = (f - f.mean(axis=1, keepdims=True)) / f.std(axis=1, keepdims=True)
        F = np.ascontiguousarray(f.T)
        qf = F + noise * rng.standard_normal((L, n_field), dtype=np.float32)
        kf = F + noise * rng.standard_normal((L, n_field), dtype=np.float32)
        q[b, h] = _to_tensor(np.concatenate([qf, loc], axis=1), dtype)
        k[b, h] = _to_tensor(np.concatenate([kf, loc], axis=1), dtype)
        v[b, h] = _to_tensor(rng.standard_normal((L, D), dtype=np.float32), dtype)

    _for_units([(b, h) for b in range(B) for h in range(nh)], unit)
    return {"q": q, "k": k, "v": v}


def paged_decode(seed: int, lens, Hq: int, Hkv: int, D: int, Dv: int, n_c: int, r: float,
                 block_size: int, dtype: str = "bf16", spare_blocks: int = 3,
                 latent: bool = False) -> dict:
    """Variable-length decode inputs in a block-paged KV cache.

    Sequence i (length ``lens[i]``) is drawn as ``clustered_decode`` with seed
    ``[seed, i]`` and one batch entry.  Its keys/values are then cut into
    ``block_size``-row blocks and written to the blocks of a shared cache
    ``[num_blocks, Hkv, block_size, D]`` in a random order (a permutation drawn
    from ``default_rng([seed, 1 << 20])``, plus ``spare_blocks`` unused blocks),
    the way a serving engine scatters pages.  Returns the cache tensors, the
    block table ``[B, max_blocks]`` (int32, -1 past a sequence's end), the
    lengths (int32), the queries ``[B, Hq, D]``, and the contiguous
    per-sequence ``k_seqs[i] [Hkv, L_i, D]`` / ``v_seqs[i]`` for a reference
    to read without any paging.  ``latent``: no V is drawn (``v_cache`` and
    ``v_seqs`` are None; the value rows are the first ``Dv`` columns of the
    key rows), as in ``clustered_decode``.
    """
    B = len(lens)
    tdt = _torch_dtype(dtype)
    seqs = [clustered_decode(int(np.random.SeedSequence([seed, i]).generate_state(1)[0] % (1 << 30)),
                             1, Hq, Hkv, int(L), D, Dv, n_c, r, latent=latent, dtype=dtype)
            for i, L in enumerate(lens)]
    nblk = [-(-int(L) // block_size) for L in lens]
    max_blocks = max(nblk)
    total = sum(nblk) + spare_blocks
    perm = np.random.default_rng([seed, 1 << 20]).permutation(total)
    k_cache = torch.zeros((total, Hkv, block_size, D), dtype=tdt)
    v_cache = None if latent else torch.zeros((total, Hkv, block_size, Dv), dtype=tdt)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    nxt = 0
    for i, L in enumerate(lens):
        n = nblk[i]
        phys = torch.from_numpy(perm[nxt:nxt + n].astype(np.int64))
        nxt += n
        table[i, :n] = phys.numpy()
        pairs = [(seqs[i]["k"][0], k_cache)] + ([] if latent else [(seqs[i]["v"][0], v_cache)])
        for src, dst in pairs:
            pad = torch.zeros((src.shape[0], n * block_size, src.shape[2]), dtype=tdt)
            pad[:, : int(L)] = src  # [Hkv, L, d] -> blocks [n, Hkv, block_size, d]
            dst.index_copy_(0, phys, pad.reshape(src.shape[0], n, block_size, src.shape[2])
                            .permute(1, 0, 2, 3).contiguous())
    return {"q": torch.cat([s_["q"] for s_ in seqs]), "k_cache": k_cache, "v_cache": v_cache,
            "block_table": torch.from_numpy(table), "seq_lens": torch.tensor(lens, dtype=torch.int32),
            "k_seqs": [s_["k"][0] for s_ in seqs],
            "v_seqs": None if latent else [s_["v"][0] for s_ in seqs]}



def gumbel_decode(seed: int, B: int, Hq: int, Hkv: int, Lk: int, D: int, Dv: int, scale: float,
                  dtype: str = "bf16", latent: bool = False) -> dict:
    """Decode inputs whose scaled scores are i.i.d. standard Gumbel.

    Draw order, from the stream of each (b, kv head): the direction ``u``
    (normal, normalised), the scores ``g ~ Gumbel(0, 1)`` [Lk], the key noise
    [Lk, D] (projected off ``u``), then V [Lk, Dv] (skipped when ``latent``:
    the value rows are then the first ``Dv`` columns of each key row).  Every
    query head of the group is ``q = u``; key ``i`` is
    ``(g_i / scale) * u + noise_i``, so ``scale * q.k_i = g_i`` up to the
    rounding of the stored values.  With ``dtype="bf16"`` the rounding moves a
    score by a few hundredths, with ``"f32"`` by ~1e-6.
    """
    g_ = Hq // Hkv
    tdt = _torch_dtype(dtype)
    q = torch.empty((B, Hq, D), dtype=tdt)
    k = torch.empty((B, Hkv, Lk, D), dtype=tdt)
    v = None if latent else torch.empty((B, Hkv, Lk, Dv), dtype=tdt)

    def unit(bh):
        b, hk = bh
        rng = _unit_rng(seed, b, hk)
        u = rng.standard_normal(D)
        u /= np.linalg.norm(u)
        g = rng.gumbel(size=Lk)
        noise = rng.standard_normal((Lk, D))
        noise -= np.outer(noise @ u, u)
        kk = (g / scale)[:, None] * u[None, :] + noise
        q[b, hk * g_:(hk + 1) * g_] = _to_tensor(np.repeat(u[None, :], g_, axis=0), dtype)
        k[b, hk] = _to_tensor(kk, dtype)
        if not latent:
            v[b, hk] = _to_tensor(rng.standard_normal((Lk, Dv), dtype=np.float32), dtype)

    _for_units([(b, hk) for b in range(B) for hk in range(Hkv)], unit)
    return {"q": q, "k": k, "v": v}


def output_gradient(seed: int, B: int, H: int, L: int, Dv: int, dtype: str = "bf16") -> torch.Tensor:
    """dL/dout for a backward call: i.i.d. N(0, 1) [B, H, L, Dv], one stream
    per (b, head) so a slice of heads draws the same values at any size."""
    out = torch.empty((B, H, L, Dv), dtype=_torch_dtype(dtype))

    def unit(bh):
        b, h = bh
        out[b, h] = _to_tensor(_unit_rng(seed, b, h).standard_normal((L, Dv), dtype=np.float32),
                               dtype)

    _for_units([(b, h) for b in range(B) for h in range(H)], unit)
    return out
