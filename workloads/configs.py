"""The five synthetic decode workloads and their seeded generators.

Shapes follow the decode workloads that the DCP pages describe: GQA models with
few KV heads and MLA models whose one latent KV head (576 = 512 latent + 64
rope dims, value = the first 512 dims) is shared by all query heads, served at
high concurrency with long, skewed contexts (median about 67K tokens in the
agent-style benchmark of the Qiita article, section "どれだけ効くか").

Everything here is input construction:

* lengths: fixed, uniform integers, or lognormal around a median;
* a page pool of exactly sum(ceil(L_b / block_size)) pages, shuffled and handed
  out to sequences in order (unused table slots hold -1);
* queries and caches drawn N(0, std) in float32, then rounded to bf16 with
  round-to-nearest-even when the workload is bf16;
* optional planted keys that make a few scores large, so that the LSE merge
  has to cope with widely separated maxima.

Seeds: workload k uses ``numpy.random.SeedSequence(1000 + k)`` (or an explicit
seed), spawned into five children: lengths, block table, queries, caches,
plants.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

KIND_GQA = "gqa"
KIND_MLA = "mla"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "gqa" or "mla"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    block_size: int
    num_shards: int
    dtype: str  # "f32" or "bf16"
    softmax_scale: float
    # length law: "fixed" (lengths), "uniform" (lo..hi inclusive) or "lognormal"
    length_law: str = "fixed"
    lengths: Optional[Sequence[int]] = None
    length_lo: int = 0
    length_hi: int = 0
    length_median: float = 0.0
    length_sigma: float = 0.0
    length_cap: Optional[int] = None
    # value laws (standard deviations). MLA: first `head_dim_v` dims use
    # std_latent, the remaining rope dims use std_rope. GQA: std_latent for all.
    std_latent: float = 1.0
    std_rope: float = 1.0
    # planted keys per (sequence, kv head); score target on the scaled logit
    plants_per_head: int = 0
    plant_score: float = 0.0
    seed_index: int = 0

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _gqa(name, **kw):
    return Workload(name=name, kind=KIND_GQA, **kw)


def _mla(name, **kw):
    base = dict(name=name, kind=KIND_MLA, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                block_size=64, num_shards=8, dtype="bf16", softmax_scale=1.0 / math.sqrt(192.0),
                length_law="lognormal", length_median=67000.0, length_sigma=0.6,
                std_latent=0.5, std_rope=1.0)
    base.update(kw)
    return Workload(**base)


WORKLOADS = {
    # 1: tiny fp32 GQA, 2 x 1024 tokens, 4 shards of 256
    "gqa-tiny": _gqa(
        "gqa-tiny", batch=2, num_q_heads=8, num_kv_heads=2, head_dim_qk=64, head_dim_v=64,
        block_size=16, num_shards=4, dtype="f32", softmax_scale=1.0 / 8.0,
        length_law="fixed", lengths=(1024, 1024), seed_index=1),
    # 2: GQA with 4 KV heads, groups of 16, contexts U[8K, 32K]
    "gqa-g16": _gqa(
        "gqa-g16", batch=32, num_q_heads=64, num_kv_heads=4, head_dim_qk=128, head_dim_v=128,
        block_size=16, num_shards=2, dtype="bf16", softmax_scale=1.0 / math.sqrt(128.0),
        length_law="uniform", length_lo=8192, length_hi=32768, seed_index=2),
    # 3: MLA, 128 heads, 64 sequences, lognormal median 67K capped at 128K
    "mla-128h": _mla("mla-128h", batch=64, num_q_heads=128, length_cap=131072, seed_index=3),
    # 4: MLA, 64 heads, 512 sequences, lognormal median 67K (the headline)
    "mla-64h-b512": _mla("mla-64h-b512", batch=512, num_q_heads=64, seed_index=4),
    # prefill chunks scored against the sharded cache (bench.py --q-len 512): MLA at the
    # agent workload's 5th / 50th / 95th percentile contexts and beyond, GQA at 32K
    "mla-prefill": _mla("mla-prefill", batch=4, num_q_heads=64, length_law="fixed",
                        lengths=(20_000, 67_000, 120_000, 180_000), seed_index=6),
    "gqa-prefill": _gqa(
        "gqa-prefill", batch=4, num_q_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
        block_size=16, num_shards=8, dtype="bf16", softmax_scale=1.0 / math.sqrt(128.0),
        length_law="fixed", lengths=(32_768, 32_768, 32_768, 32_768), seed_index=7),
    # 5: very long GQA contexts with planted high-score keys
    "gqa-long": _gqa(
        "gqa-long", batch=4, num_q_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
        block_size=16, num_shards=16, dtype="bf16", softmax_scale=1.0 / math.sqrt(128.0),
        length_law="fixed", lengths=(200_000, 500_000, 800_000, 1_000_000),
        plants_per_head=3, plant_score=20.0, seed_index=5),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _children(wl: Workload, seed: Optional[int]):
    ss = np.random.SeedSequence(1000 + wl.seed_index if seed is None else seed)
    return ss.spawn(5)


def draw_lengths(wl: Workload, ss: np.random.SeedSequence) -> np.ndarray:
    """Context lengths L_b (int64), per the workload's length law."""
    rng = np.random.default_rng(ss)
    if wl.length_law == "fixed":
        lens = np.asarray(wl.lengths, dtype=np.int64)
        assert lens.shape == (wl.batch,)
    elif wl.length_law == "uniform":
        lens = rng.integers(wl.length_lo, wl.length_hi, size=wl.batch, endpoint=True)
    elif wl.length_law == "lognormal":
        z = rng.standard_normal(wl.batch)
        lens = np.rint(np.exp(math.log(wl.length_median) + wl.length_sigma * z)).astype(np.int64)
        if wl.length_cap is not None:
            lens = np.minimum(lens, wl.length_cap)
        lens = np.maximum(lens, 1)
    else:
        raise ValueError(wl.length_law)
    return lens.astype(np.int64)


def draw_block_table(lengths: np.ndarray, block_size: int, ss, max_blocks: Optional[int] = None):
    """Shuffled page pool handed out to sequences in order.

    Returns (block_table int32 [B, max_blocks] with -1 in unused slots,
    num_blocks). The pool holds exactly sum_b ceil(L_b / block_size) pages.
    """
    rng = np.random.default_rng(ss)
    need = [(int(L) + block_size - 1) // block_size for L in lengths]
    num_blocks = max(1, int(sum(need)))
    if max_blocks is None:
        max_blocks = max(1, max(need) if need else 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(lengths), max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, num_blocks


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def _f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _std_vector(wl: Workload) -> np.ndarray:
    std = np.full(wl.head_dim_qk, wl.std_latent, dtype=np.float32)
    if wl.kind == KIND_MLA:
        std[wl.head_dim_v:] = wl.std_rope
    return std


def _plant_positions(L: int, block_size: int, count: int, rng) -> list:
    """Three kinds of positions: near the end, a page start, anywhere."""
    out = []
    for j in range(count):
        if j % 3 == 0:
            out.append(L - 1 - int(rng.integers(0, max(1, L // 32))))
        elif j % 3 == 1:
            npages = (L + block_size - 1) // block_size
            out.append(min(L - 1, int(rng.integers(0, npages)) * block_size))
        else:
            out.append(int(rng.integers(0, L)))
    return out


def _planted_key(q_rows_f32: np.ndarray, target: float, scale: float) -> np.ndarray:
    """Key k = c * mean(q) with c chosen so that scale * <mean(q), k> = target."""
    qbar = q_rows_f32.astype(np.float64).mean(axis=0)
    c = target / (scale * float(qbar @ qbar))
    return (c * qbar).astype(np.float32)


def make_host_inputs(wl: Workload, seed: Optional[int] = None, lengths=None, max_blocks=None):
    """Draw every input on the host with numpy.

    Returns a dict: seq_lens int32 [B], block_table int32 [B, max_blocks],
    num_blocks, q [B, Hq, Dqk], and either k_cache/v_cache [num_blocks, Hkv,
    bs, D] (GQA) or kv_cache [num_blocks, bs, Dqk] (MLA). bf16 arrays are
    uint16 bit patterns; f32 arrays are float32.
    """
    c_len, c_tab, c_q, c_kv, c_plant = _children(wl, seed)
    lens = np.asarray(lengths, dtype=np.int64) if lengths is not None else draw_lengths(wl, c_len)
    table, num_blocks = draw_block_table(lens, wl.block_size, c_tab, max_blocks)
    std = _std_vector(wl)
    rq = np.random.default_rng(c_q)
    q32 = (rq.standard_normal((wl.batch, wl.num_q_heads, wl.head_dim_qk), dtype=np.float32) * std)
    rkv = np.random.default_rng(c_kv)
    bs = wl.block_size
    if wl.kind == KIND_MLA:
        kv32 = rkv.standard_normal((num_blocks, bs, wl.head_dim_qk), dtype=np.float32) * std
        caches = {"kv_cache": kv32}
    else:
        shape = (num_blocks, wl.num_kv_heads, bs, wl.head_dim_qk)
        k32 = rkv.standard_normal(shape, dtype=np.float32) * std
        v32 = rkv.standard_normal(shape, dtype=np.float32) * std
        caches = {"k_cache": k32, "v_cache": v32}
    out = {"seq_lens": lens.astype(np.int32), "block_table": table, "num_blocks": num_blocks}
    if wl.dtype == "bf16":
        out["q"] = bf16_bits_from_f32(q32)
        for k, v in caches.items():
            out[k] = bf16_bits_from_f32(v)
    else:
        out["q"] = q32
        out.update(caches)
    if wl.plants_per_head:
        _plant_host(wl, out, c_plant)
    return out


def make_queries(wl: Workload, q_len: int, seed: Optional[int] = None,
                 batch: Optional[int] = None) -> np.ndarray:
    """Queries of q_len tokens per request, [B, q_len, Hq, Dqk], drawn like the one-token
    queries (bf16 as uint16 bit patterns, f32 as float32)."""
    B = wl.batch if batch is None else batch
    rng = np.random.default_rng(np.random.SeedSequence(3000 + wl.seed_index if seed is None
                                                       else seed))
    q = rng.standard_normal((B, q_len, wl.num_q_heads, wl.head_dim_qk),
                            dtype=np.float32) * _std_vector(wl)
    return bf16_bits_from_f32(q) if wl.dtype == "bf16" else q


def make_new_rows(wl: Workload, seed: Optional[int] = None, batch: Optional[int] = None):
    """Rows of the token each request decodes this step, drawn like the cache rows.

    GQA: {"new_k": [B, Hkv, Dqk], "new_v": [B, Hkv, Dv]}; MLA: {"new_latent": [B, Dqk]}.
    bf16 arrays are uint16 bit patterns, f32 arrays float32.
    """
    B = wl.batch if batch is None else batch
    rng = np.random.default_rng(np.random.SeedSequence(2000 + wl.seed_index if seed is None
                                                       else seed))
    std = _std_vector(wl)
    if wl.kind == KIND_MLA:
        rows = {"new_latent": rng.standard_normal((B, wl.head_dim_qk), dtype=np.float32) * std}
    else:
        rows = {"new_k": rng.standard_normal((B, wl.num_kv_heads, wl.head_dim_qk),
                                             dtype=np.float32) * std,
                "new_v": rng.standard_normal((B, wl.num_kv_heads, wl.head_dim_v),
                                             dtype=np.float32) * std[:wl.head_dim_v]}
    if wl.dtype == "bf16":
        rows = {k: bf16_bits_from_f32(v) for k, v in rows.items()}
    return rows


def _plant_host(wl: Workload, inp: dict, ss) -> None:
    rng = np.random.default_rng(ss)
    is_bf16 = wl.dtype == "bf16"
    q = inp["q"]
    qf = _f32_from_bf16_bits(q) if is_bf16 else q
    G = wl.group_size
    bs = wl.block_size
    plants = []
    for b in range(wl.batch):
        L = int(inp["seq_lens"][b])
        if L == 0:
            continue
        for g in range(wl.num_kv_heads):
            key = _planted_key(qf[b, g * G:(g + 1) * G], wl.plant_score, wl.softmax_scale)
            for t in _plant_positions(L, bs, wl.plants_per_head, rng):
                page = int(inp["block_table"][b, t // bs])
                row = bf16_bits_from_f32(key) if is_bf16 else key
                if wl.kind == KIND_MLA:
                    inp["kv_cache"][page, t % bs, :] = row
                else:
                    inp["k_cache"][page, g, t % bs, :] = row
                plants.append((b, g, t))
    inp["plants"] = plants


def make_device_inputs(wl: Workload, device, seed: Optional[int] = None, lengths=None,
                       chunk_elems: int = 1 << 27, max_blocks=None):
    """Draw the inputs with lengths/tables from numpy and values from torch on `device`.

    Values come from ``torch.Generator(device)`` seeded from the spawned
    children, drawn N(0, 1) in float32 chunk by chunk, scaled by the per-dim
    std and cast to the workload dtype (bf16 casts round to nearest even).
    Returns torch tensors (seq_lens and block_table are int32 on `device`;
    host copies are under seq_lens_host / block_table_host).
    """
    import torch

    c_len, c_tab, c_q, c_kv, c_plant = _children(wl, seed)
    lens = np.asarray(lengths, dtype=np.int64) if lengths is not None else draw_lengths(wl, c_len)
    table, num_blocks = draw_block_table(lens, wl.block_size, c_tab, max_blocks)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    std = torch.from_numpy(_std_vector(wl)).to(device)

    def seeded(ss):
        gen = torch.Generator(device=device)
        gen.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
        return gen

    gq = seeded(c_q)
    q = (torch.randn((wl.batch, wl.num_q_heads, wl.head_dim_qk), generator=gq, device=device,
                     dtype=torch.float32) * std).to(tdt)
    gkv = seeded(c_kv)
    bs = wl.block_size

    def fill(dst):
        per_block = dst[0].numel()
        step = max(1, chunk_elems // per_block)
        for p0 in range(0, dst.shape[0], step):
            p1 = min(dst.shape[0], p0 + step)
            tmp = torch.randn((p1 - p0,) + tuple(dst.shape[1:]), generator=gkv, device=device,
                              dtype=torch.float32)
            tmp.mul_(std)
            dst[p0:p1].copy_(tmp)
            del tmp

    out = {"seq_lens_host": lens.astype(np.int32), "block_table_host": table,
           "num_blocks": num_blocks, "q": q}
    if wl.kind == KIND_MLA:
        kv = torch.empty((num_blocks, bs, wl.head_dim_qk), dtype=tdt, device=device)
        fill(kv)
        out["kv_cache"] = kv
    else:
        shape = (num_blocks, wl.num_kv_heads, bs, wl.head_dim_qk)
        k = torch.empty(shape, dtype=tdt, device=device)
        v = torch.empty(shape, dtype=tdt, device=device)
        fill(k)
        fill(v)
        out["k_cache"] = k
        out["v_cache"] = v
    out["seq_lens"] = torch.from_numpy(lens.astype(np.int32)).to(device)
    out["block_table"] = torch.from_numpy(table).to(device)
    if wl.plants_per_head:
        rng = np.random.default_rng(c_plant)
        qf = q.float().cpu().numpy()
        G = wl.group_size
        plants = []
        for b in range(wl.batch):
            L = int(lens[b])
            if L == 0:
                continue
            for g in range(wl.num_kv_heads):
                key = torch.from_numpy(_planted_key(qf[b, g * G:(g + 1) * G], wl.plant_score,
                                                    wl.softmax_scale)).to(device).to(tdt)
                for t in _plant_positions(L, bs, wl.plants_per_head, rng):
                    page = int(table[b, t // bs])
                    if wl.kind == KIND_MLA:
                        out["kv_cache"][page, t % bs, :] = key
                    else:
                        out["k_cache"][page, g, t % bs, :] = key
                    plants.append((b, g, t))
        out["plants"] = plants
    return out
