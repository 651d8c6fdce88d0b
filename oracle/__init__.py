"""CPU oracle for selected-token sparse attention with KV append.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's
``cpu_baseline`` leg are the only callers; the product library never imports
this package, and this package never imports the product.

Two independent statements of the computation live here:

* ``sa_oracle.c`` (loaded through ctypes): the plain fp32 definition with the
  pages' strictly ascending reductions -- append, index validation, forward,
  and the fp8_e4m3_block64 record codec. Sources: the IndexShare CUDA kernel
  page (onnx-runtime-ep-cuda ``src/kernels/index_share.rs``: ``index_share_row``,
  host ``validate_indices``) and the CSA CPU oracle page (onnx-runtime-ep-cpu
  ``src/kernels/compressed_sparse_attention.rs``: ``CacheFormat``,
  ``dequantize_cache``, ``dot`` / ``accumulate_value``).
* ``textbook_attention`` (numpy float64): dense softmax attention with an
  optional boolean mask and softcap, written as the textbook formula. It pins
  the C forward (all-selected rows must agree to fp32 rounding).

Pins for every function are in ``tests/test_oracle_*.py``; none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "sa_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None
_lock = threading.Lock()

# storage codes used by sa_oracle.c
F32, F16, BF16, FP8_BLOCK64 = 0, 1, 2, 3
SEPARATE, SHARED_LATENT = 0, 1
CLASS_NAMES = {0: "ok", 1: "sentinel", 2: "after_padding", 3: "range", 4: "duplicate",
               5: "order", 6: "all_padding"}

_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11", "-Wall"]


def build(force: bool = True) -> Path:
    """Compile sa_oracle.c with gcc (no FMA contraction, no fast-math)."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.run(["gcc", *_CFLAGS, str(_SRC), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        lib = ctypes.CDLL(str(_LIB_PATH))
        P, I64, U8P = ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint8)
        lib.oracle_bf16_from_f32.argtypes = [ctypes.c_float]
        lib.oracle_bf16_from_f32.restype = ctypes.c_uint16
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3fn_value.restype = ctypes.c_double
        lib.oracle_fp8_quantize_block64.argtypes = [P, P, P]
        lib.oracle_fp8_quantize_block64.restype = ctypes.c_int
        lib.oracle_fp8_record_bytes.argtypes = [I64, I64]
        lib.oracle_fp8_record_bytes.restype = I64
        lib.oracle_fp8_pack_record.argtypes = [P, I64, I64, P]
        lib.oracle_fp8_pack_record.restype = ctypes.c_int
        lib.oracle_fp8_decode_record.argtypes = [P, I64, I64, P]
        lib.oracle_fp8_decode_record.restype = ctypes.c_int
        lib.oracle_kv_append.argtypes = [P, I64, P, P, I64, P, I64, I64, I64, I64]
        lib.oracle_kv_append.restype = ctypes.c_int
        lib.oracle_validate_indices.argtypes = [P, ctypes.c_int, I64, I64, I64, I64, P, U8P,
                                                P, P, P, ctypes.c_char_p, I64]
        lib.oracle_validate_indices.restype = ctypes.c_uint32
        lib.oracle_forward_rows.argtypes = [P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, I64,
                                            P, ctypes.c_int, I64, I64, I64, I64, I64, I64, I64, I64,
                                            I64, ctypes.c_float, ctypes.c_float, P, ctypes.c_int, P,
                                            I64, I64, P, P]
        lib.oracle_forward_rows.restype = ctypes.c_int
        lib.oracle_capacity_lengths.argtypes = [P, ctypes.c_int, P, I64, I64, I64, I64, I64, P, P]
        lib.oracle_capacity_lengths.restype = None
        lib.oracle_csa_sink_attention.argtypes = [P, I64, I64, I64, P, I64, P, I64, P, I64, I64,
                                                  P, P, P, I64, ctypes.c_float, P]
        lib.oracle_csa_sink_attention.restype = ctypes.c_uint32
        lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_value.restype = ctypes.c_double
        lib.oracle_fp4_quantize_block32.argtypes = [P, P, P, P]
        lib.oracle_fp4_quantize_block32.restype = ctypes.c_int
        lib.oracle_fp4_decode_key.argtypes = [P, I64, P]
        lib.oracle_fp4_decode_key.restype = None
        lib.oracle_compressed_rope.argtypes = [P, I64, I64]
        lib.oracle_compressed_rope.restype = None
        lib.oracle_hadamard_f32.argtypes = [P, I64]
        lib.oracle_hadamard_f32.restype = None
        lib.oracle_finalize_index_query.argtypes = [P, I64, I64, I64, P]
        lib.oracle_finalize_index_query.restype = ctypes.c_int
        lib.oracle_csa_index_select.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, P, P]
        lib.oracle_csa_index_select.restype = ctypes.c_uint32
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- scalars
def bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bits, nearest-even (oracle rounding, one value at a time)."""
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_bf16_from_f32(float(flat_in[i]))
    return out


def bf16_round_f32(x) -> np.ndarray:
    """fp32 values rounded to bf16 (nearest-even) and widened back."""
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


def f16_to_f32(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> fp32 values (the oracle's widening of f16 inputs)."""
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    flat_in, flat_out = b.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_f16_to_f32(int(flat_in[i]))
    return out


def e4m3fn_value(code: int) -> float:
    return _load().oracle_e4m3fn_value(code)


def e8m0_value(byte: int) -> float:
    return _load().oracle_e8m0_value(byte)


# ---------------------------------------------------------------- fp8 records
def fp8_record_bytes(dk: int, rope: int) -> int:
    return int(_load().oracle_fp8_record_bytes(dk, rope))


def fp8_quantize_block64(x) -> tuple[int, np.ndarray]:
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(64)
    scale = np.zeros(1, np.uint8)
    codes = np.zeros(64, np.uint8)
    if _load().oracle_fp8_quantize_block64(_ptr(x), _ptr(scale), _ptr(codes)) != 0:
        raise ValueError("fp8 quantizer: non-finite value in block")
    return int(scale[0]), codes


def fp8_pack_rows(rows, rope: int) -> np.ndarray:
    """[..., Dk] fp32 logical rows -> [..., record_bytes] uint8 records."""
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    dk = rows.shape[-1]
    rb = fp8_record_bytes(dk, rope)
    if rb < 0:
        raise ValueError("(Dk - rope) must be a multiple of 64")
    flat = rows.reshape(-1, dk)
    out = np.empty((flat.shape[0], rb), np.uint8)
    lib = _load()
    for i in range(flat.shape[0]):
        if lib.oracle_fp8_pack_record(_ptr(flat[i]), dk, rope, _ptr(out[i])) != 0:
            raise ValueError("fp8 record pack: non-finite value")
    return out.reshape(rows.shape[:-1] + (rb,))


def fp8_decode_rows(records, dk: int, rope: int) -> np.ndarray:
    records = np.ascontiguousarray(records, dtype=np.uint8)
    rb = records.shape[-1]
    flat = records.reshape(-1, rb)
    out = np.empty((flat.shape[0], dk), np.float32)
    lib = _load()
    for i in range(flat.shape[0]):
        if lib.oracle_fp8_decode_record(_ptr(flat[i]), dk, rope, _ptr(out[i])) != 0:
            raise ValueError("fp8 record decode: NaN scale or code")
    return out.reshape(records.shape[:-1] + (dk,))


# ---------------------------------------------------------------- A1 append
def kv_append(past: np.ndarray, past_len, cur: np.ndarray, present: np.ndarray | None = None):
    """Byte-level append. past/present [B, H, cap, row...]; cur [B, H, C, row...].

    present=None means in place (present aliases past); returns present."""
    past = np.ascontiguousarray(past)
    in_place = present is None
    if in_place:
        present = past
    cur = np.ascontiguousarray(cur)
    assert past.dtype == cur.dtype == present.dtype
    B, H, pcap = past.shape[:3]
    C = cur.shape[2]
    row_bytes = int(np.prod(past.shape[3:], dtype=np.int64)) * past.dtype.itemsize
    plen = np.ascontiguousarray(past_len, dtype=np.int64).reshape(B)
    rc = _load().oracle_kv_append(_ptr(past), pcap, _ptr(plen), _ptr(cur), C, _ptr(present),
                                  present.shape[2], B, H, row_bytes)
    if rc != 0:
        raise ValueError("kv_append: past_len + cur_len exceeds capacity")
    return present


# ---------------------------------------------------------------- A3 validate
class IndexError_(ValueError):
    pass


def validate_indices(indices: np.ndarray, bound, *, raise_first: bool = False):
    """indices [B, Hi, Sq, W] int32/int64; bound [B] cache length per batch.

    Returns (word, row_class[B*Hi*Sq] uint8, (row, col, cls) of the first
    failure or None, message)."""
    idx = np.ascontiguousarray(indices)
    assert idx.dtype in (np.int32, np.int64) and idx.ndim == 4
    B, Hi, Sq, W = idx.shape
    bnd = np.ascontiguousarray(bound, dtype=np.int64).reshape(B)
    row_class = np.zeros(B * Hi * Sq, np.uint8)
    fr, fc, fk = (np.zeros(1, np.int64), np.zeros(1, np.int64), np.zeros(1, np.int32))
    msg = ctypes.create_string_buffer(512)
    word = _load().oracle_validate_indices(
        _ptr(idx), int(idx.dtype == np.int64), B, Hi, Sq, W, _ptr(bnd),
        row_class.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), _ptr(fr), _ptr(fc), _ptr(fk),
        msg, 512)
    first = None if fr[0] < 0 else (int(fr[0]), int(fc[0]), int(fk[0]))
    text = msg.value.decode()
    if raise_first and first is not None:
        raise IndexError_(text)
    return int(word), row_class, first, text


# ---------------------------------------------------------------- forward
def bias_dims(shape, keys=None) -> np.ndarray:
    """A bias shape of rank <= 4 right-aligned against [B, H, S, keys] and
    padded with 1 on the left (int64[4])."""
    shape = tuple(int(d) for d in shape)
    if len(shape) > 4:
        raise ValueError(f"attention_bias rank {len(shape)} exceeds 4")
    return np.array((1,) * (4 - len(shape)) + shape, np.int64)


def capacity_lengths(bias, keys: int, cur_len: int, *, batch: int, heads: int, q_seq: int,
                     bias_dtype: int = 0):
    """Capacity-mode length recovery (oracle C `oracle_capacity_lengths`):
    per batch, valid = 1 + the last key column where the bias is finite for
    any (head, query), and write_pos = valid - cur_len (0 below cur_len).
    bias holds raw storage of bias_dtype (float32, or uint16 bits)."""
    bias = np.ascontiguousarray(bias)
    dims = bias_dims(bias.shape)
    valid = np.zeros(batch, np.int64)
    wpos = np.zeros(batch, np.int64)
    _load().oracle_capacity_lengths(_ptr(bias), bias_dtype, _ptr(dims), batch, heads, q_seq, keys,
                                    cur_len, _ptr(valid), _ptr(wpos))
    return valid, wpos


def forward(q, kcache, vcache, indices, *, q_dtype: int, cache_fmt: int, kv_layout: int,
            hkv: int, dv: int, rope: int = 0, scale: float = 0.0, softcap: float = 0.0,
            bias=None, bias_dtype: int | None = None,
            rows=None, threads: int | None = None) -> np.ndarray:
    """Oracle forward. Arrays hold raw storage (bf16/f16 as uint16 bits, fp8 as
    uint8 records). q [B, Hq, Sq, Dk]; kcache [B, Hkv, cap, Dk or record];
    vcache [B, Hkv, cap, Dv] or None; indices [B, Hi, Sq, W].
    bias: None, or an additive bias of rank <= 4 broadcast right-aligned
    against [B, Hq, Sq, cap] (raw storage of bias_dtype, default q_dtype),
    indexed by the selected key's cache position and added after the softcap.

    rows: None for all output rows, or an iterable of flattened (b, h, q) row
    ids -- only those rows of the returned fp32 [B*Hq*Sq, Dv] array are set.
    threads: rows are spread over this many Python threads (each C call
    releases the GIL); every row keeps its own ascending order."""
    lib = _load()
    q = np.ascontiguousarray(q)
    kcache = np.ascontiguousarray(kcache)
    if vcache is not None:
        vcache = np.ascontiguousarray(vcache)
    idx = np.ascontiguousarray(indices)
    B, Hq, Sq, Dk = q.shape
    cap = kcache.shape[2]
    Hi, W = idx.shape[1], idx.shape[3]
    total = B * Hq * Sq
    bdims = None
    if bias is not None:
        bias = np.ascontiguousarray(bias)
        bdims = bias_dims(bias.shape)
        for a, t in enumerate((B, Hq, Sq, cap)):
            if bdims[a] not in (1, t):
                raise ValueError(f"attention_bias shape {bias.shape} is not broadcastable to {(B, Hq, Sq, cap)}")
        bias_dtype = q_dtype if bias_dtype is None else bias_dtype
    y = np.zeros((total, dv), np.float32)
    row_list = np.arange(total, dtype=np.int64) if rows is None else np.asarray(list(rows), np.int64)
    nthreads = max(1, min(threads or 1, len(row_list)))
    errors = []

    def run(chunk):
        work = np.empty(2 * max(Dk, dv) + W, np.float32)
        # contiguous runs are passed as one range
        start = 0
        while start < len(chunk):
            end = start + 1
            while end < len(chunk) and chunk[end] == chunk[end - 1] + 1:
                end += 1
            rc = lib.oracle_forward_rows(
                _ptr(q), q_dtype, _ptr(kcache), None if vcache is None else _ptr(vcache),
                cache_fmt, kv_layout, cap, _ptr(idx), int(idx.dtype == np.int64), B, Hq, hkv, Sq,
                Hi, W, Dk, dv, rope, float(scale), float(softcap),
                None if bias is None else _ptr(bias), 0 if bias is None else int(bias_dtype),
                None if bdims is None else _ptr(bdims), int(chunk[start]),
                int(chunk[end - 1]) + 1, _ptr(y), _ptr(work))
            if rc != 0:
                errors.append(rc)
                return
            start = end

    if nthreads == 1:
        run(row_list)
    else:
        parts = np.array_split(row_list, nthreads)
        ts = [threading.Thread(target=run, args=(p,)) for p in parts]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    if errors:
        raise ValueError("oracle forward: index out of range or NaN record")
    return y.reshape(B, Hq, Sq, dv)


# ---------------------------------------------------------------- CSA sink attention
CSA_DIM, CSA_ROPE, CSA_RECORD_BYTES, CSA_WINDOW = 512, 64, 583, 128
CSA_RANGE, CSA_DENOM, CSA_GEOMETRY = 1, 2, 4


def csa_sink_attention(query, current_kv, records, selected, sink, total: int, *,
                       scale: float = 0.0, bias=None):
    """CSA ratio-4 selected sink attention (oracle C `oracle_csa_sink_attention`).

    query [B, S, H, 512] fp32; current_kv [B, Tcur, 512] fp32; records
    [B, Rcap, 583] uint8; selected [B, Hidx, S, K] int32 (index head 0 read);
    sink [H] fp32; bias None or fp32 of rank <= 4 broadcastable to
    [B, H, S, Cd + K]. Returns (y [B, S, H, 512] fp32, flags)."""
    lib = _load()
    q = np.ascontiguousarray(query, np.float32)
    ckv = np.ascontiguousarray(current_kv, np.float32)
    rec = np.ascontiguousarray(records, np.uint8)
    sel = np.ascontiguousarray(selected, np.int32)
    snk = np.ascontiguousarray(sink, np.float32)
    B, S, H, D = q.shape
    assert D == CSA_DIM and ckv.shape[0] == B and ckv.shape[2] == D
    assert rec.shape[0] == B and rec.shape[2] == CSA_RECORD_BYTES
    assert sel.ndim == 4 and sel.shape[0] == B and sel.shape[2] == S and snk.shape == (H,)
    dims = np.ones(4, np.int64)
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, np.float32)
        assert b.ndim <= 4
        if b.ndim:
            dims[4 - b.ndim:] = b.shape
    y = np.zeros((B, S, H, D), np.float32)
    flags = lib.oracle_csa_sink_attention(
        _ptr(q), B, S, H, _ptr(ckv), ckv.shape[1], _ptr(rec), rec.shape[1], _ptr(sel), sel.shape[1],
        sel.shape[3], _ptr(snk), None if b is None else _ptr(b), _ptr(dims), int(total),
        float(scale), _ptr(y))
    if flags == 0xFFFFFFFF:
        raise MemoryError("oracle csa_sink_attention: allocation failed")
    return y, int(flags)


# ---------------------------------------------------------------- CSA selection producer
SEL_NONFINITE, SEL_TIE, SEL_GEOMETRY = 1, 2, 4


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(code)


def fp4_quantize_block32(x):
    """32 fp32 values -> (scale byte, 16 packed bytes, dequantized fp32[32])."""
    x = np.ascontiguousarray(x, np.float32)
    assert x.shape == (32,)
    sc, packed, out = np.zeros(1, np.uint8), np.zeros(16, np.uint8), np.zeros(32, np.float32)
    if _load().oracle_fp4_quantize_block32(_ptr(x), _ptr(sc), _ptr(packed), _ptr(out)) != 0:
        raise ValueError("fp4 quantize: non-finite value")
    return int(sc[0]), packed, out


def fp4_pack_keys(rows) -> np.ndarray:
    """[..., dim] fp32 -> [..., dim/32*17] FP4 index keys (blocks of scale + 16 bytes)."""
    rows = np.ascontiguousarray(rows, np.float32)
    dim = rows.shape[-1]
    flat = rows.reshape(-1, dim)
    out = np.zeros((flat.shape[0], dim // 32 * 17), np.uint8)
    for i in range(flat.shape[0]):
        for b in range(dim // 32):
            sc, packed, _ = fp4_quantize_block32(flat[i, 32 * b:32 * b + 32])
            out[i, 17 * b] = sc
            out[i, 17 * b + 1:17 * b + 17] = packed
    return out.reshape(rows.shape[:-1] + (dim // 32 * 17,))


def fp4_decode_keys(keys, dim: int) -> np.ndarray:
    keys = np.ascontiguousarray(keys, np.uint8)
    flat = keys.reshape(-1, keys.shape[-1])
    out = np.empty((flat.shape[0], dim), np.float32)
    lib = _load()
    for i in range(flat.shape[0]):
        lib.oracle_fp4_decode_key(_ptr(flat[i]), dim, _ptr(out[i]))
    return out.reshape(keys.shape[:-1] + (dim,))


def compressed_rope(tail, position: int) -> np.ndarray:
    t = np.array(tail, np.float32, copy=True)
    _load().oracle_compressed_rope(_ptr(t), t.shape[0], int(position))
    return t


def hadamard_f32(v) -> np.ndarray:
    t = np.array(v, np.float32, copy=True)
    _load().oracle_hadamard_f32(_ptr(t), t.shape[0])
    return t


def finalize_index_query(src, rope: int, position: int) -> np.ndarray:
    src = np.ascontiguousarray(src, np.float32)
    q = np.empty_like(src)
    if _load().oracle_finalize_index_query(_ptr(src), src.shape[0], rope, int(position), _ptr(q)) != 0:
        raise ValueError("finalize_index_query: non-finite value")
    return q


def csa_index_select(index_query, index_weight, index_keys, total: int, topk: int, *, rope: int = 64,
                     with_scores: bool = False):
    """index_query [B, S, H, dim] fp32, index_weight [B, S, H] fp32, index_keys
    [B, Rcap, dim/32*17] uint8. Returns (selected [B, S, topk] int32, flags[, scores
    [B, S, Rcap] fp32 with NaN past each query's causal records])."""
    iq = np.ascontiguousarray(index_query, np.float32)
    iw = np.ascontiguousarray(index_weight, np.float32)
    keys = np.ascontiguousarray(index_keys, np.uint8)
    B, S, H, dim = iq.shape
    assert iw.shape == (B, S, H) and keys.shape[0] == B and keys.shape[2] == dim // 32 * 17
    sel = np.full((B, S, topk), -1, np.int32)
    scores = np.empty((B, S, keys.shape[1]), np.float32) if with_scores else None
    flags = _load().oracle_csa_index_select(_ptr(iq), _ptr(iw), _ptr(keys), B, S, H, dim, rope, keys.shape[1],
                                            int(total), int(topk), _ptr(sel),
                                            None if scores is None else _ptr(scores))
    if flags == 0xFFFFFFFF:
        raise MemoryError("oracle csa_index_select: allocation failed")
    return (sel, int(flags), scores) if with_scores else (sel, int(flags))


# ---------------------------------------------------------------- textbook
def textbook_attention(q, k, v, *, scale: float, mask=None, softcap: float = 0.0) -> np.ndarray:
    """Dense softmax attention in float64: softmax(softcap(scale * Q K^T) + mask) V.

    q [..., M, D]; k [..., N, D]; v [..., N, Dv]; mask [..., M, N] boolean
    (True = attend). Rows with no attended key are zero."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * scale
    if softcap:
        s = softcap * np.tanh(s / softcap)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - safe_m)
    den = np.sum(e, axis=-1, keepdims=True)
    p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
    return np.matmul(p, v)
