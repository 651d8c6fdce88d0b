"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the oracle on the same seeded inputs. Expected values come only from the
oracle (and from the input generator); nothing read back from the device is
ever fed to the oracle."""
from __future__ import annotations

import numpy as np

import oracle
import sa_workloads as W

# tolerance of the floating outputs: |y - y_oracle| <= ATOL + RTOL * |y_oracle|
TOL = {W.DT_F32: (1e-5, 0.0), W.DT_F16: (2e-2, 1e-2), W.DT_BF16: (2e-2, 1e-2)}


def torch_mod():
    import torch
    return torch


def tt(a):
    """Host array -> device tensor (16-bit patterns travel as int16)."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def fill_garbage(t):
    """Finite garbage in spare cache rows (7.5 / -4.25 style): a read of them shows."""
    torch = torch_mod()
    if t.dtype == torch.float32:
        t.fill_(-4.25)
    elif t.dtype == torch.int16:
        t.fill_(0x4121)   # bf16 10.0625
    else:
        t.fill_(0x5A)
    return t


def raw_bytes(a):
    return np.ascontiguousarray(a).view(np.uint8)


def to_np(t):
    return t.detach().cpu().numpy()


def y_as_f32(t):
    torch = torch_mod()
    if t.dtype == torch.float32:
        return to_np(t)
    return to_np(t.float())


def y_dtype(w):
    torch = torch_mod()
    return {W.DT_F32: torch.float32, W.DT_F16: torch.float16, W.DT_BF16: torch.bfloat16}[w.dtype]


def make_ctx(w, *, idx64=False, max_batch=None, max_q_seq=None, max_width=None, max_cap=None,
             softcap=None):
    import sparse_attention_kv_append_amd as sa
    return sa.Context(num_heads=w.hq, kv_num_heads=w.hkv, head_dim_qk=w.dk, head_dim_v=w.dv,
                      dtype=w.dtype, kv_layout=w.layout,
                      cache_format=(sa.SA_CACHE_FP8_E4M3_BLOCK64 if w.cache_format == W.CACHE_FP8
                                    else sa.SA_CACHE_DENSE),
                      rope_dim=w.rope, index_dtype=sa.SA_IDX_I64 if idx64 else sa.SA_IDX_I32,
                      scale=w.scale, softcap=w.softcap if softcap is None else softcap,
                      max_batch=max_batch or w.batch, max_q_seq=max_q_seq or w.q_seq,
                      max_index_width=max_width or w.width, max_cache_len=max_cap or w.cap)


def check_close(y, ref, dtype, what=""):
    atol, rtol = TOL[dtype]
    err = np.abs(y.astype(np.float64) - ref.astype(np.float64))
    bound = atol + rtol * np.abs(ref.astype(np.float64))
    bad = err > bound
    assert not np.isnan(y).any(), f"{what}: NaN in device output"
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance; max err "
                           f"{err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())


def oracle_present(inp):
    """Oracle append of the generator's past and current rows (in place)."""
    pk = oracle.kv_append(inp["past_k"].copy(), inp["past_len"], inp["cur_k"])
    pv = None
    if inp["past_v"] is not None:
        pv = oracle.kv_append(inp["past_v"].copy(), inp["past_len"], inp["cur_v"])
    return pk, pv


def oracle_records(rows_bits, w):
    """fp8 records (oracle quantizer) of bf16 rows given as uint16 bits."""
    f32 = (rows_bits.astype(np.uint32) << 16).view(np.float32)
    return oracle.fp8_pack_rows(f32, w.rope)


def run_device(w, inp, *, mode="inplace", idx64=False, fused=True, fp8_cur="records",
               indices=None, ctx=None, records=None):
    """Append + forward on the device. Returns (y_f32, present_k, present_v,
    error_word). For fp8 workloads the past cache is the oracle's records of
    the generator's bf16 rows and the current rows are given either as
    oracle records (byte append) or as bf16 rows (quantized on the device)."""
    torch = torch_mod()
    own = ctx is None
    if own:
        ctx = make_ctx(w, idx64=idx64)
    B, H = w.batch, w.hkv
    fp8 = w.cache_format == W.CACHE_FP8
    if fp8 and records is not None:
        past_host, cur_host = records  # caller-built records (planted bytes)
    elif fp8:
        past_host = oracle_records(inp["past_k"], w)
        cur_host = inp["cur_k"] if fp8_cur == "bf16" else oracle_records(inp["cur_k"], w)
    else:
        past_host = inp["past_k"]
        cur_host = inp["cur_k"]
    idx_host = inp["indices"] if indices is None else indices
    if idx64:
        idx_host = idx_host.astype(np.int64)
    plen = tt(inp["past_len"])
    vlen = torch.full_like(plen, -7)
    cap = w.cap
    if mode == "inplace":
        kc = tt(past_host)
        vc = tt(inp["past_v"]) if inp["past_v"] is not None else None
        pk_dev, pv_dev = kc, vc
        past_k_arg, past_v_arg, past_cap = kc, vc, cap
    else:  # concat into fresh buffers filled with garbage
        kc = tt(np.ascontiguousarray(past_host[:, :, :w.past]))
        vc = tt(np.ascontiguousarray(inp["past_v"][:, :, :w.past])) if inp["past_v"] is not None else None
        pk_dev = fill_garbage(torch.empty((B, H, cap) + tuple(past_host.shape[3:]), dtype=kc.dtype,
                                          device="cuda"))
        pv_dev = None
        if vc is not None:
            pv_dev = fill_garbage(torch.empty((B, H, cap, w.dv), dtype=vc.dtype, device="cuda"))
        past_k_arg, past_v_arg, past_cap = kc, vc, w.past
    before_k = to_np(pk_dev)
    before_v = None if pv_dev is None else to_np(pv_dev)
    cur_k = tt(cur_host)
    cur_v = tt(inp["cur_v"]) if inp["cur_v"] is not None else None
    ctx.reset_error_async()
    ctx.kv_append(B, past_k_arg if past_cap > 0 else None, past_v_arg if past_cap > 0 else None,
                  past_cap, plen, cur_k, cur_v, w.cur, pk_dev, pv_dev, cap,
                  cur_is_unquantized_bf16=(fp8 and fp8_cur == "bf16"), present_len=vlen)
    y = torch.full((B, w.hq, w.q_seq, w.dv), float("nan"), dtype=y_dtype(w), device="cuda")
    ctx.forward(tt(inp["q"]), B, w.q_seq, pk_dev, pv_dev, cap, vlen, tt(idx_host),
                idx_host.shape[1], idx_host.shape[3], y, fused_validate=fused)
    word, fb, msg = ctx.read_error()
    out = dict(y=y_as_f32(y), present_k=to_np(pk_dev), present_v=None if pv_dev is None else to_np(pv_dev),
               word=word, first_bad=fb, msg=msg, valid_len=to_np(vlen), before_k=before_k,
               before_v=before_v)
    if own:
        ctx.destroy()
    return out


def check_present(w, dev, pk_ref, pv_ref):
    """Rows below the valid length equal the oracle's present bit for bit;
    spare capacity rows still hold what the present buffer held before."""
    T = w.total
    for got, ref, before in ((dev["present_k"], pk_ref, dev["before_k"]),
                             (dev["present_v"], pv_ref, dev["before_v"])):
        if ref is None:
            continue
        assert np.array_equal(raw_bytes(got[:, :, :T]), raw_bytes(ref[:, :, :T]))
        assert np.array_equal(raw_bytes(got[:, :, T:]), raw_bytes(before[:, :, T:]))


def run_oracle(w, inp, indices=None, threads=8, records=None):
    """Oracle append + forward. Returns (y, present_k, present_v) where
    present_k is records for fp8 workloads (records: caller-built
    (past, current) records appended as bytes)."""
    pk, pv = oracle_present(inp)
    fmt = w.dtype
    kcache = pk
    if w.cache_format == W.CACHE_FP8:
        if records is not None:
            kcache = oracle.kv_append(records[0].copy(), inp["past_len"], records[1])
        else:
            kcache = oracle_records(pk, w)
        fmt = oracle.FP8_BLOCK64
    idx = inp["indices"] if indices is None else indices
    y = oracle.forward(inp["q"], kcache, pv, idx, q_dtype=w.dtype, cache_fmt=fmt,
                       kv_layout=w.layout, hkv=w.hkv, dv=w.dv, rope=w.rope, scale=w.scale,
                       softcap=w.softcap, threads=threads)
    return y, kcache, pv
