"""Seeded synthetic inputs for selected-token sparse attention with KV append.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, and it is the one piece that the oracle side and the
device side share. Storage conventions: bf16 and f16 tensors are returned as
their raw 16-bit patterns (uint16), f32 as float32, indices as int32.

Draw order for every workload (numpy ``default_rng(seed)``): Q, then the past
cache (K then V, or the single shared-latent cache), then the current rows,
then the index rows in (batch, index_head, query) order. Normal draws are
fp32 N(0, 1); bf16 values are torch's round-to-nearest-even cast of them.

Workloads (sizes are the ones the pages' operators are exercised at; the
"scaled" variants keep the structure at sizes the CPU oracle finishes fast):

* ``tiny_f32``     batch 1, 4 q heads / 4 kv heads, head dim 64, past 60 +
                   4 current, 4 query rows each selecting 16 sorted distinct
                   keys from [0, 64), width 20 with trailing -1; f32; scale 1/8.
* ``decode_bf16``  batch 32, 1 query, 64 q heads sharing 1 kv head, shared
                   latent rows of 576 (512 latent + 64 rope; V = first 512),
                   past 32768 + 1 current, top-2048 uniform without
                   replacement from [0, 32769), sorted; bf16.
* ``decode_fp8``   as decode_bf16 with batch 64, past 65536 + 1; the cache is
                   fp8_e4m3_block64 records (made by a block quantizer from
                   the bf16 values this module returns).
* ``prefill_bf16`` batch 1, empty past, 4096 current = query rows, 64 q heads
                   sharing 1 kv head, row i selects min(i+1, 2048) sorted keys
                   of [0, i] (all of them below 2048), width 2048.
* ``dense_gqa``    batch 8, 32 q heads / 8 kv heads, head dim 128, past 8064 +
                   128 current, 128 query rows; row q selects every key of
                   [0, 8064 + q] (causal with per-batch offset 8064), width
                   8192; softcap 50; bf16.
* ``gqa_decode_b2`` batch 2, 32 q heads / 8 kv heads, head dim 128, past
                   32767 + 1 current, 1 query, top-8192 uniform sorted; bf16
                   (few (batch, kv head) pairs: the split-KV decode).

Capacity mode with an attention bias (``CAPACITY_WORKLOADS``, drawn by
``make_capacity_numpy``): separate K and V caches of ``capacity`` rows per
(batch, kv head) drawn in full (rows past the live length hold stale values
that must not be read), then the current rows; per batch entry a live length
valid_b uniform over [valid_lo, capacity]; then the bias [B, 1, Sq,
capacity], N(0, 1) * 0.5 up to the query's position and -inf after it (the
causal/padding frontier that carries valid_b); then index rows as
``causal_prefill`` against valid_b (query s sits at position valid_b - Sq + s).

* ``capacity_small``  batch 3, 8 q heads / 2 kv heads, head dim 64, 2 queries
                      and 2 current rows, capacity 300, top-40 of width 48; f32.
* ``capacity_decode`` batch 32, 32 q heads / 8 kv heads, head dim 128, 1 query
                      and 1 current row, capacity 16384, live lengths
                      8192..16384, top-2048; bf16.

CSA ratio-4 sink attention (``CSA_WORKLOADS``, drawn by ``make_csa_numpy``):
query [B, S, H, 512] and current_kv [B, Tcur, 512] fp32 N(0, 1); the record
source rows [B, total/4, 512] N(0, 1) rounded to bf16 (a block quantizer turns
them into 583-byte records); head_sink [H] N(0, 1); query s (position
total - S + s) selects min(K, (pos + 1) // 4) distinct complete records drawn
uniformly, in random order (the order a top-k by score leaves), padded with
-1 and repeated over the index heads.

* ``csa_small``    batch 2, 3 queries, 32 heads, Tcur 140, total 300, K 40.
* ``csa_decode``   batch 64, 1 query, 64 heads, Tcur 128, total 65536 (16384
                   records per batch entry), K 512.

CSA selection producer (``CSA_INDEX_WORKLOADS``, ``make_csa_index_numpy``):
index queries [B, S, H, 128] and weights [B, S, H] fp32 N(0, 1); FP4 index
keys [B, key_cap, 68] drawn as bytes: every code nibble uniform over the 16
E2M1 codes, every block's scale byte uniform over 122..126.

* ``csa_index_small``  batch 2, 3 queries, 16 index heads, 300 keys, total 900, K 40.
* ``csa_index_decode`` batch 64, 1 query, 64 index heads, 16384 keys, total
                       65536, K 512.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

DT_F32, DT_F16, DT_BF16 = 0, 1, 2
LAYOUT_SEPARATE, LAYOUT_SHARED_LATENT = 0, 1
CACHE_DENSE, CACHE_FP8 = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    q_seq: int
    dk: int
    dv: int
    past: int          # past length of every batch entry
    cur: int           # current rows appended this step
    width: int         # index row width
    topk: int          # selected keys per row (before any per-row cap)
    dtype: int         # DT_*
    layout: int        # LAYOUT_*
    cache_format: int  # CACHE_*
    rope: int = 0
    scale: float = 0.0     # 0 -> 1/sqrt(dk)
    softcap: float = 0.0
    index_heads: int = 1
    pattern: str = "uniform"   # uniform | causal_prefill | causal_all
    seed: int = 0
    capacity: int = 0          # cache rows allocated per (b, kv head); 0 -> past + cur
    extra: dict = field(default_factory=dict)

    @property
    def cap(self) -> int:
        return self.capacity or (self.past + self.cur)

    @property
    def total(self) -> int:
        return self.past + self.cur

    @property
    def rows(self) -> int:
        return self.batch * self.hq * self.q_seq

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", batch=1, hq=4, hkv=4, q_seq=4, dk=64, dv=64, past=60, cur=4,
                         width=20, topk=16, dtype=DT_F32, layout=LAYOUT_SEPARATE,
                         cache_format=CACHE_DENSE, scale=1.0 / 8.0, seed=0),
    "decode_bf16": Workload("decode_bf16", batch=32, hq=64, hkv=1, q_seq=1, dk=576, dv=512,
                            past=32768, cur=1, width=2048, topk=2048, dtype=DT_BF16,
                            layout=LAYOUT_SHARED_LATENT, cache_format=CACHE_DENSE, rope=64,
                            scale=1.0 / 24.0, seed=1),
    "decode_fp8": Workload("decode_fp8", batch=64, hq=64, hkv=1, q_seq=1, dk=576, dv=512,
                           past=65536, cur=1, width=2048, topk=2048, dtype=DT_BF16,
                           layout=LAYOUT_SHARED_LATENT, cache_format=CACHE_FP8, rope=64,
                           scale=1.0 / 24.0, seed=2),
    "prefill_bf16": Workload("prefill_bf16", batch=1, hq=64, hkv=1, q_seq=4096, dk=576, dv=512,
                             past=0, cur=4096, width=2048, topk=2048, dtype=DT_BF16,
                             layout=LAYOUT_SHARED_LATENT, cache_format=CACHE_DENSE, rope=64,
                             scale=1.0 / 24.0, pattern="causal_prefill", seed=3),
    # a prefill with more query rows than the eight-wave kernel addresses
    # (63 head strides of q_seq rows must fit 32 bits): the four-wave kernel
    "prefill_long_q": Workload("prefill_long_q", batch=1, hq=64, hkv=1, q_seq=29700, dk=576, dv=512, past=0,
                               cur=29700, width=16, topk=16, dtype=DT_BF16, layout=LAYOUT_SHARED_LATENT,
                               cache_format=CACHE_DENSE, rope=64, scale=1.0 / 24.0, pattern="causal_prefill",
                               seed=6),
    "dense_gqa": Workload("dense_gqa", batch=8, hq=32, hkv=8, q_seq=128, dk=128, dv=128,
                          past=8064, cur=128, width=8192, topk=8192, dtype=DT_BF16,
                          layout=LAYOUT_SEPARATE, cache_format=CACHE_DENSE,
                          scale=float(1.0 / np.sqrt(np.float32(128.0))), softcap=50.0,
                          pattern="causal_all", seed=4),
    "gqa_decode_b2": Workload("gqa_decode_b2", batch=2, hq=32, hkv=8, q_seq=1, dk=128, dv=128,
                              past=32767, cur=1, width=8192, topk=8192, dtype=DT_BF16,
                              layout=LAYOUT_SEPARATE, cache_format=CACHE_DENSE,
                              scale=float(1.0 / np.sqrt(np.float32(128.0))), seed=7),
}


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _store(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == DT_F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == DT_F16:
        return _f16_bits(x)
    return _bf16_bits(x)


def index_rows(w: Workload, rng: np.random.Generator, bound=None) -> np.ndarray:
    """[B, Hi, Sq, W] int32 index rows for workload `w` (draws in row order)."""
    B, Hi, Sq, W = w.batch, w.index_heads, w.q_seq, w.width
    bound = np.full(B, w.total, np.int64) if bound is None else np.asarray(bound, np.int64)
    out = np.full((B, Hi, Sq, W), -1, np.int32)
    for b in range(B):
        T = int(bound[b])
        for h in range(Hi):
            for q in range(Sq):
                if w.pattern == "uniform":
                    k = min(w.topk, T, W)
                    sel = np.sort(rng.choice(T, size=k, replace=False))
                elif w.pattern == "causal_prefill":
                    # query row q is at absolute position (T - Sq) + q
                    pos = T - Sq + q
                    avail = pos + 1
                    if avail <= w.topk:
                        sel = np.arange(avail)
                    else:
                        sel = np.sort(rng.choice(avail, size=w.topk, replace=False))
                elif w.pattern == "causal_all":
                    pos = T - Sq + q
                    sel = np.arange(min(pos + 1, W))
                else:
                    raise ValueError(w.pattern)
                out[b, h, q, :len(sel)] = sel
    return out


def make_numpy(w: Workload) -> dict:
    """All inputs of workload `w`, drawn on the host.

    Returns q, past_k, past_v (None for shared latent), cur_k, cur_v, indices,
    past_len, valid_len and, for shared-latent workloads, the logical fp32
    latent values (``past_kv_f32``/``cur_kv_f32``) that fp8 records encode."""
    rng = np.random.default_rng(w.seed)
    B, Hq, Hkv, Sq, Dk, Dv = w.batch, w.hq, w.hkv, w.q_seq, w.dk, w.dv
    q32 = rng.standard_normal((B, Hq, Sq, Dk), dtype=np.float32)
    out = {"workload": w, "q": _store(q32, w.dtype)}
    cap = w.cap
    if w.layout == LAYOUT_SEPARATE:
        pk = rng.standard_normal((B, Hkv, w.past, Dk), dtype=np.float32)
        pv = rng.standard_normal((B, Hkv, w.past, Dv), dtype=np.float32)
        ck = rng.standard_normal((B, Hkv, w.cur, Dk), dtype=np.float32)
        cv = rng.standard_normal((B, Hkv, w.cur, Dv), dtype=np.float32)
        out["past_k"] = _pad_cap(_store(pk, w.dtype), cap)
        out["past_v"] = _pad_cap(_store(pv, w.dtype), cap)
        out["cur_k"] = _store(ck, w.dtype)
        out["cur_v"] = _store(cv, w.dtype)
    else:
        pkv = rng.standard_normal((B, Hkv, w.past, Dk), dtype=np.float32)
        ckv = rng.standard_normal((B, Hkv, w.cur, Dk), dtype=np.float32)
        pkv_b = _store(pkv, w.dtype)
        ckv_b = _store(ckv, w.dtype)
        out["past_k"] = _pad_cap(pkv_b, cap)
        out["past_v"] = None
        out["cur_k"] = ckv_b
        out["cur_v"] = None
        # logical values the cache rows hold (bf16 widened), for fp8 packing
        out["past_kv_f32"] = _widen(pkv_b, w.dtype)
        out["cur_kv_f32"] = _widen(ckv_b, w.dtype)
    out["past_len"] = np.full(B, w.past, np.int32)
    out["valid_len"] = np.full(B, w.total, np.int32)
    out["indices"] = index_rows(w, rng)
    return out


CAPACITY_WORKLOADS = {
    "capacity_small": Workload("capacity_small", batch=3, hq=8, hkv=2, q_seq=2, dk=64, dv=64, past=0, cur=2,
                               width=48, topk=40, dtype=DT_F32, layout=LAYOUT_SEPARATE,
                               cache_format=CACHE_DENSE, scale=1.0 / 8.0, pattern="causal_prefill",
                               seed=5, capacity=300, extra={"valid_lo": 2}),
    "capacity_decode": Workload("capacity_decode", batch=32, hq=32, hkv=8, q_seq=1, dk=128, dv=128, past=0,
                                cur=1, width=2048, topk=2048, dtype=DT_BF16, layout=LAYOUT_SEPARATE,
                                cache_format=CACHE_DENSE, scale=float(1.0 / np.sqrt(np.float32(128.0))),
                                pattern="causal_prefill", seed=6, capacity=16384,
                                extra={"valid_lo": 8192}),
    # the decode_bf16 shapes (64 heads over one 576-dim shared-latent row of
    # which the first 512 dims are V) in capacity mode
    "capacity_latent_decode": Workload("capacity_latent_decode", batch=32, hq=64, hkv=1, q_seq=1, dk=576,
                                       dv=512, past=0, cur=1, width=2048, topk=2048, dtype=DT_BF16,
                                       layout=LAYOUT_SHARED_LATENT, cache_format=CACHE_DENSE,
                                       scale=float(1.0 / np.sqrt(np.float32(576.0))), pattern="causal_prefill",
                                       seed=7, capacity=32769, extra={"valid_lo": 16384}),
}


def make_capacity_numpy(w: Workload) -> dict:
    """Inputs of a capacity-mode workload: q, past_k, past_v (all capacity
    rows), cur_k, cur_v, valid (int64 [B], the live length after this step),
    indices, bias (config dtype storage, [B, 1, Sq, capacity])."""
    rng = np.random.default_rng(w.seed)
    B, Hq, Hkv, Sq, Dk, Dv, cap = w.batch, w.hq, w.hkv, w.q_seq, w.dk, w.dv, w.cap
    out = {"workload": w}
    out["q"] = _store(rng.standard_normal((B, Hq, Sq, Dk), dtype=np.float32), w.dtype)
    out["past_k"] = _store(rng.standard_normal((B, Hkv, cap, Dk), dtype=np.float32), w.dtype)
    out["past_v"] = _store(rng.standard_normal((B, Hkv, cap, Dv), dtype=np.float32), w.dtype)
    out["cur_k"] = _store(rng.standard_normal((B, Hkv, w.cur, Dk), dtype=np.float32), w.dtype)
    out["cur_v"] = _store(rng.standard_normal((B, Hkv, w.cur, Dv), dtype=np.float32), w.dtype)
    valid, bias = capacity_frontier(w, rng)
    out["valid"] = valid
    out["bias_f32"] = bias
    out["bias"] = _store(bias, w.dtype)
    out["indices"] = index_rows(w, rng, bound=valid)
    return out


def capacity_frontier(w: Workload, rng: np.random.Generator):
    """Live lengths valid [B] (int64, uniform over [valid_lo, capacity]) and
    the fp32 bias [B, 1, Sq, capacity]: N(0, 1) * 0.5 up to query s's
    position valid_b - Sq + s, -inf after it."""
    B, Sq, cap = w.batch, w.q_seq, w.cap
    lo = max(int(w.extra["valid_lo"]), w.cur, Sq)
    valid = rng.integers(lo, cap + 1, B).astype(np.int64)
    bias = (rng.standard_normal((B, 1, Sq, cap), dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    for b in range(B):
        for s in range(Sq):
            bias[b, 0, s, valid[b] - Sq + s + 1:] = -np.inf
    return valid, bias


def store_elems(x: np.ndarray, dtype: int) -> np.ndarray:
    """fp32 values -> storage of dtype (bf16/f16 as uint16 bits, RNE)."""
    return _store(x, dtype)


def _widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Storage -> fp32 by reinterpretation (bf16: bits << 16). Layout only."""
    if dtype == DT_F32:
        return bits.astype(np.float32)
    if dtype == DT_F16:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _pad_cap(a: np.ndarray, cap: int) -> np.ndarray:
    """Place [B, H, past, ...] into a [B, H, cap, ...] buffer; spare rows get
    finite garbage (7.5 / -4.25 patterns) so a read of them shows."""
    B, H, P = a.shape[:3]
    if cap == P:
        return np.ascontiguousarray(a)
    out = np.empty((B, H, cap) + a.shape[3:], a.dtype)
    out[:, :, :P] = a
    if a.dtype == np.float32:
        garbage = np.float32(7.5)
    elif a.dtype == np.uint16:
        garbage = np.uint16(0x40F0)  # 7.5 in bf16
    else:
        garbage = a.dtype.type(0x55)
    out[:, :, P:] = garbage
    return out


def torch_normal_f32(shape, seed: int, device: str = "cuda"):
    """N(0,1) fp32 tensors drawn on the device with a seeded torch generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def torch_normal_bf16(shape, seed: int, device: str = "cuda"):
    """Large N(0,1) bf16 tensors drawn on the device with a seeded torch
    generator (for the full-size decode caches, too large to draw on the host)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


@dataclass(frozen=True)
class CsaWorkload:
    name: str
    batch: int
    seq: int
    heads: int
    cur_len: int        # current_kv rows (absolute positions total - cur_len ..)
    total: int          # total_sequence_length
    topk: int           # selected_indices width K
    index_heads: int = 1
    record_cap: int = 0  # record rows allocated per batch entry; 0 -> total // 4
    seed: int = 0
    scale: float = 0.0   # 0 -> 1/sqrt(512)

    @property
    def records(self) -> int:
        return self.total // 4

    @property
    def cap(self) -> int:
        return self.record_cap or self.records

    def scaled(self, **kw) -> "CsaWorkload":
        return replace(self, **kw)


CSA_DIM = 512
CSA_WORKLOADS = {
    "csa_small": CsaWorkload("csa_small", batch=2, seq=3, heads=32, cur_len=140, total=300,
                             topk=40, index_heads=2, seed=20),
    "csa_decode": CsaWorkload("csa_decode", batch=64, seq=1, heads=64, cur_len=128, total=65536,
                              topk=512, seed=21),
}


def csa_selection(w: CsaWorkload, rng: np.random.Generator) -> np.ndarray:
    """[B, Hidx, S, K] int32: per query, distinct complete records in random order."""
    B, S, K = w.batch, w.seq, w.topk
    out = np.full((B, w.index_heads, S, K), -1, np.int32)
    for b in range(B):
        for s in range(S):
            pos = w.total - S + s
            avail = (pos + 1) // 4
            k = min(K, avail)
            if k > 0:
                out[b, :, s, :k] = rng.choice(avail, size=k, replace=False)
    return out


def make_csa_numpy(w: CsaWorkload) -> dict:
    """Host inputs of a CSA workload: query, current_kv, record_rows (fp32
    values, bf16-representable, [B, total/4, 512]), sink, selected."""
    rng = np.random.default_rng(w.seed)
    B, S, H = w.batch, w.seq, w.heads
    q = rng.standard_normal((B, S, H, CSA_DIM), dtype=np.float32)
    ckv = rng.standard_normal((B, w.cur_len, CSA_DIM), dtype=np.float32)
    rows = rng.standard_normal((B, w.records, CSA_DIM), dtype=np.float32)
    rows = _widen(_bf16_bits(rows), DT_BF16)
    sink = rng.standard_normal(H, dtype=np.float32)
    sel = csa_selection(w, rng)
    return {"workload": w, "query": q, "current_kv": ckv, "record_rows": rows, "sink": sink,
            "selected": sel}


@dataclass(frozen=True)
class CsaIndexWorkload:
    name: str
    batch: int
    seq: int
    heads: int
    key_cap: int
    total: int
    topk: int
    out_heads: int = 1
    seed: int = 0

    def scaled(self, **kw) -> "CsaIndexWorkload":
        return replace(self, **kw)


CSA_INDEX_WORKLOADS = {
    "csa_index_small": CsaIndexWorkload("csa_index_small", batch=2, seq=3, heads=16, key_cap=300, total=900,
                                        topk=40, out_heads=2, seed=30),
    "csa_index_decode": CsaIndexWorkload("csa_index_decode", batch=64, seq=1, heads=64, key_cap=16384,
                                         total=65536, topk=512, seed=31),
}


def csa_index_keys(rng: np.random.Generator, batch: int, key_cap: int) -> np.ndarray:
    """[B, key_cap, 68] FP4 index keys as random bytes (codes uniform, scale bytes 122..126)."""
    keys = rng.integers(0, 256, (batch, key_cap, 68), dtype=np.uint8)
    keys[:, :, 0::17] = rng.integers(122, 127, (batch, key_cap, 4), dtype=np.uint8)
    return keys


def make_csa_index_numpy(w: CsaIndexWorkload) -> dict:
    rng = np.random.default_rng(w.seed)
    iq = rng.standard_normal((w.batch, w.seq, w.heads, 128), dtype=np.float32)
    iw = rng.standard_normal((w.batch, w.seq, w.heads), dtype=np.float32)
    keys = csa_index_keys(rng, w.batch, w.key_cap)
    return {"workload": w, "index_query": iq, "index_weight": iw, "index_keys": keys}
