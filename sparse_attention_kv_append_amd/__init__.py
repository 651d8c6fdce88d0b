"""Python binding of libsparse_attn.so (selected-token sparse attention with KV
append on MI355X / gfx950).

The binding only marshals arguments: every step of the path runs in the HIP
kernels of the shared library. torch supplies device memory and the stream.
If the library is not built, importing the ``native`` handle raises -- there
is no fallback implementation of any step.

The C entry points are exposed under their own names (``sparse_attn_create``,
``sparse_attn_kv_append``, ...) taking raw pointers and sizes, and the
``Context`` class wraps them for torch tensors.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "libsparse_attn.so"

# ---- constants mirrored from include/sparse_attn.h
SA_OK, SA_E_ARG, SA_E_SHAPE, SA_E_DTYPE, SA_E_CAPACITY, SA_E_UNSUPPORTED, SA_E_HIP, SA_E_STATE, \
    SA_E_INDEX = range(9)
SA_F32, SA_F16, SA_BF16 = 0, 1, 2
SA_CACHE_DENSE, SA_CACHE_FP8_E4M3_BLOCK64 = 0, 1
SA_KV_SEPARATE, SA_KV_SHARED_LATENT = 0, 1
SA_IDX_I32, SA_IDX_I64 = 0, 1
SA_ERR_SENTINEL, SA_ERR_AFTER_PAD, SA_ERR_RANGE = 0x01, 0x02, 0x04
SA_ERR_DUPLICATE, SA_ERR_ORDER, SA_ERR_ALL_PAD = 0x08, 0x10, 0x20
SA_ERR_APPEND_CAPACITY, SA_ERR_QUANT_NONFINITE = 0x40, 0x80
SA_ERR_INDEX_ANY, SA_ERR_APPEND_ANY = 512, 1024
SA_STATIC_SCRATCH_BYTES = 48 << 20
SA_ERR_CSA_GEOMETRY, SA_ERR_CSA_DENOM, SA_ERR_INDEX_NONFINITE = 0x100, 0x800, 0x1000
SA_ERR_INDEX_TIE = 0x2000
SA_PEAK_READ_SINK_WORDS = 1024 * 256

STATUS_NAMES = {0: "SA_OK", 1: "SA_E_ARG", 2: "SA_E_SHAPE", 3: "SA_E_DTYPE", 4: "SA_E_CAPACITY",
                5: "SA_E_UNSUPPORTED", 6: "SA_E_HIP", 7: "SA_E_STATE", 8: "SA_E_INDEX"}

EXPORTS = [
    "sparse_attn_create", "sparse_attn_destroy", "sparse_attn_set_stream",
    "sparse_attn_kv_append", "sparse_attn_validate_indices", "sparse_attn_forward", "sparse_attn_step",
    "sparse_attn_forward_bias", "sparse_attn_capacity_lengths", "sparse_attn_capacity_step",
    "sparse_attn_csa_forward", "sparse_attn_csa_index_select", "sparse_attn_csa_index_workspace_bytes",
    "sparse_attn_reset_error_async", "sparse_attn_read_error", "sparse_attn_last_error",
    "sparse_attn_query_plan", "sparse_attn_profile_enable", "sparse_attn_profile_read",
    "sparse_attn_version", "sparse_attn_forward_latent_static",
    "sparse_attn_measure_copy", "sparse_attn_measure_read", "sparse_attn_measure_mfma", "sparse_attn_step_kv",
]


class sa_config(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32), ("kv_num_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("cache_format", ctypes.c_int32), ("kv_layout", ctypes.c_int32),
        ("index_dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("softcap", ctypes.c_float),
        ("max_batch", ctypes.c_int64), ("max_q_seq", ctypes.c_int64),
        ("max_index_width", ctypes.c_int64), ("max_cache_len", ctypes.c_int64),
    ]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def load(path: Path | str | None = None) -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(
            f"{p} is missing: build the HIP library first (python -m "
            "sparse_attention_kv_append_amd.build or __graft_entry__.build())")
    # torch ships its own HIP runtime (soname libamdhip64.so.7) and loads it by
    # a name that does not match an already loaded system copy; loaded first,
    # it is the one this library binds to, so the process keeps one runtime
    import torch  # noqa: F401
    lib = ctypes.CDLL(str(p))
    V, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    st = ctypes.c_int
    sig = {
        "sparse_attn_create": ([ctypes.POINTER(sa_config), V, ctypes.POINTER(V)], st),
        "sparse_attn_destroy": ([V], st),
        "sparse_attn_set_stream": ([V, V], st),
        "sparse_attn_kv_append": ([V, I64, V, V, I64, V, V, V, I64, I32, V, V, I64, V], st),
        "sparse_attn_validate_indices": ([V, V, I64, I64, I64, I64, V, I64, V, V, V], st),
        "sparse_attn_forward": ([V, V, I64, I64, V, V, I64, V, V, I64, I64, V, I32], st),
        "sparse_attn_forward_bias": ([V, V, I64, I64, V, V, I64, V, V, I64, I64, V, V, I32, V, I32], st),
        "sparse_attn_capacity_lengths": ([V, V, V, I32, I64, I64, I64, I64, V, V], st),
        "sparse_attn_capacity_step": ([V, V, I64, I64, V, V, I64, V, V, I64, V, I64, I64, V, V, I32, V, V, V, I32],
                                      st),
        "sparse_attn_step": ([V, V, I64, I64, V, I64, V, V, I64, I32, V, V, I64, I64, V, I32], st),
        "sparse_attn_step_kv": ([V, V, I64, I64, V, V, I64, V, V, V, I64, V, V, I64, I64, V, I32], st),
        "sparse_attn_csa_forward": ([V, V, I64, I64, I64, V, I64, V, I64, V, I64, I64, V, V, V, V,
                                     ctypes.c_float, V], st),
        "sparse_attn_csa_index_select": ([V, V, V, V, I64, I64, I64, I64, V, I64, I64, V, V], st),
        "sparse_attn_csa_index_workspace_bytes": ([I64, I64, I64, I64], ctypes.c_size_t),
        "sparse_attn_reset_error_async": ([V], st),
        "sparse_attn_read_error": ([V, ctypes.POINTER(ctypes.c_uint32),
                                    ctypes.POINTER(ctypes.c_uint64)], st),
        "sparse_attn_last_error": ([V], ctypes.c_char_p),
        "sparse_attn_query_plan": ([V, I64, I64, I64, I64, ctypes.POINTER(I32),
                                    ctypes.POINTER(I32)], st),
        "sparse_attn_profile_enable": ([V, I32], st),
        "sparse_attn_profile_read": ([V, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)], st),
        "sparse_attn_version": ([], ctypes.c_char_p),
        "sparse_attn_forward_latent_static": ([V, I64, I64, V, I64, V, V, I32, I64, ctypes.c_float,
                                               ctypes.c_float, V, V], st),
        "sparse_attn_measure_copy": ([V, V, V, I64], st),
        "sparse_attn_measure_read": ([V, V, V, I64], st),
        "sparse_attn_measure_mfma": ([V, V, I64, I32], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Context:
    """One library context (config, device error word, split-K buffers).

    Methods launch on the torch stream current at call time."""

    def __init__(self, *, num_heads, kv_num_heads, head_dim_qk, head_dim_v, dtype,
                 kv_layout=SA_KV_SEPARATE, cache_format=SA_CACHE_DENSE, rope_dim=0,
                 index_dtype=SA_IDX_I32, scale=0.0, softcap=0.0, max_batch=1, max_q_seq=1,
                 max_index_width=1, max_cache_len=1):
        self.lib = load()
        self.cfg = sa_config(num_heads, kv_num_heads, head_dim_qk, head_dim_v, rope_dim, dtype,
                             cache_format, kv_layout, index_dtype, scale, softcap, max_batch,
                             max_q_seq, max_index_width, max_cache_len)
        h = ctypes.c_void_p()
        st = self.lib.sparse_attn_create(ctypes.byref(self.cfg), _stream_handle(), ctypes.byref(h))
        if st != SA_OK:
            raise SparseAttnError(st, "sparse_attn_create rejected the configuration")
        self.handle = h.value

    # -- plumbing
    def _sync_stream(self):
        self.lib.sparse_attn_set_stream(self.handle, _stream_handle())

    def _check(self, st):
        if st != SA_OK:
            raise SparseAttnError(st, self.last_error())

    def last_error(self) -> str:
        return self.lib.sparse_attn_last_error(self.handle).decode()

    def destroy(self):
        if self.handle:
            self.lib.sparse_attn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    # -- entry points
    def kv_append(self, batch, past_k, past_v, past_capacity, past_len, cur_k, cur_v, cur_len,
                  present_k, present_v, present_capacity, *, cur_is_unquantized_bf16=False,
                  present_len=None):
        self._sync_stream()
        self._check(self.lib.sparse_attn_kv_append(
            self.handle, batch, _ptr(past_k), _ptr(past_v), past_capacity, _ptr(past_len),
            _ptr(cur_k), _ptr(cur_v), cur_len, int(cur_is_unquantized_bf16), _ptr(present_k),
            _ptr(present_v), present_capacity, _ptr(present_len)))

    def validate_indices(self, indices, batch, index_heads, q_seq, width, valid_len=None,
                         cache_len=0, error_word=None, row_class=None, first_bad=None):
        self._sync_stream()
        self._check(self.lib.sparse_attn_validate_indices(
            self.handle, _ptr(indices), batch, index_heads, q_seq, width, _ptr(valid_len),
            cache_len, _ptr(error_word), _ptr(row_class), _ptr(first_bad)))

    def forward(self, q, batch, q_seq, present_k, present_v, cache_capacity, valid_len, indices,
                index_heads, width, y, fused_validate=False):
        self._sync_stream()
        self._check(self.lib.sparse_attn_forward(
            self.handle, _ptr(q), batch, q_seq, _ptr(present_k), _ptr(present_v), cache_capacity,
            _ptr(valid_len), _ptr(indices), index_heads, width, _ptr(y), int(fused_validate)))

    def forward_bias(self, q, batch, q_seq, present_k, present_v, cache_capacity, valid_len, indices,
                     index_heads, width, bias, y, fused_validate=False):
        """forward with the optional additive attention_bias (a dense tensor of
        the config dtype, rank <= 4, broadcast against [B, Hq, Sq, cache_capacity])."""
        self._sync_stream()
        dims = [] if bias is None else [int(d) for d in bias.shape]
        rank = len(dims)
        shape = (ctypes.c_int64 * max(4, rank))(*dims)
        self._check(self.lib.sparse_attn_forward_bias(
            self.handle, _ptr(q), batch, q_seq, _ptr(present_k), _ptr(present_v), cache_capacity,
            _ptr(valid_len), _ptr(indices), index_heads, width, _ptr(bias), shape, rank, _ptr(y),
            int(fused_validate)))

    def capacity_lengths(self, bias, batch, q_seq, cache_capacity, cur_len, valid_len, write_pos):
        """Capacity-mode length recovery from the bias frontier into device
        int32 [B] valid_len and write_pos."""
        self._sync_stream()
        dims = [int(d) for d in bias.shape]
        shape = (ctypes.c_int64 * max(4, len(dims)))(*dims)
        self._check(self.lib.sparse_attn_capacity_lengths(
            self.handle, _ptr(bias), shape, len(dims), batch, q_seq, cache_capacity, cur_len,
            _ptr(valid_len), _ptr(write_pos)))

    def capacity_step(self, q, batch, q_seq, cache_k, cache_v, cache_capacity, cur_k, cur_v, cur_len, indices,
                      index_heads, width, bias, y, valid_len, write_pos, reset_error=True):
        """Capacity-mode step over separate K/V caches: lengths from the bias,
        in-place append at the write position, biased forward with fused
        validation."""
        self._sync_stream()
        dims = [int(d) for d in bias.shape]
        shape = (ctypes.c_int64 * max(4, len(dims)))(*dims)
        self._check(self.lib.sparse_attn_capacity_step(
            self.handle, _ptr(q), batch, q_seq, _ptr(cache_k), _ptr(cache_v), cache_capacity, _ptr(cur_k),
            _ptr(cur_v), cur_len, _ptr(indices), index_heads, width, _ptr(bias), shape, len(dims), _ptr(y),
            _ptr(valid_len), _ptr(write_pos), int(reset_error)))

    def step(self, q, batch, q_seq, cache, cache_capacity, past_len, cur, cur_len, present_len, indices,
             index_heads, width, y, reset_error=True, cur_is_unquantized_bf16=False):
        """Reset (optional) + in-place append + forward with fused validation
        on a shared-latent cache, one launch where the library can."""
        self._sync_stream()
        self._check(self.lib.sparse_attn_step(
            self.handle, _ptr(q), batch, q_seq, _ptr(cache), cache_capacity, _ptr(past_len), _ptr(cur),
            cur_len, int(cur_is_unquantized_bf16), _ptr(present_len), _ptr(indices), index_heads, width,
            _ptr(y), int(reset_error)))

    def step_kv(self, q, batch, q_seq, cache_k, cache_v, cache_capacity, past_len, cur_k, cur_v, cur_len,
                present_len, indices, index_heads, width, y, reset_error=True):
        """Reset (optional) + in-place append + forward with fused validation
        on separate K/V caches, one launch on the grouped-query path."""
        self._sync_stream()
        self._check(self.lib.sparse_attn_step_kv(
            self.handle, _ptr(q), batch, q_seq, _ptr(cache_k), _ptr(cache_v), cache_capacity, _ptr(past_len),
            _ptr(cur_k), _ptr(cur_v), cur_len, _ptr(present_len), _ptr(indices), index_heads, width, _ptr(y),
            int(reset_error)))

    def csa_forward(self, query, current_kv, records, selected, head_sink, total_len, y, *,
                    scale=0.0, bias=None):
        """CSA ratio-4 selected sink attention. query [B, S, H, 512] f32,
        current_kv [B, Tcur, 512] f32, records [B, Rcap, 583] u8, selected
        [B, Hidx, S, K] i32, head_sink [H] f32, total_len int64 device tensor
        of one element, y [B, S, H, 512] f32, bias None or f32 of rank <= 4."""
        B, S, H, _ = query.shape
        bias_dims = None
        if bias is not None:
            dims = [1] * (4 - bias.dim()) + list(bias.shape)
            bias_dims = (ctypes.c_int64 * 4)(*dims)
        self._sync_stream()
        self._check(self.lib.sparse_attn_csa_forward(
            self.handle, _ptr(query), B, S, H, _ptr(current_kv), current_kv.shape[1], _ptr(records),
            records.shape[1], _ptr(selected), selected.shape[1], selected.shape[3], _ptr(head_sink),
            _ptr(bias), None if bias_dims is None else ctypes.cast(bias_dims, ctypes.c_void_p),
            _ptr(total_len), float(scale), _ptr(y)))

    def csa_index_workspace_bytes(self, batch, q_seq, heads, key_cap):
        return int(self.lib.sparse_attn_csa_index_workspace_bytes(batch, q_seq, heads, key_cap))

    def csa_index_select(self, index_query, index_weight, index_keys, total_len, selected, workspace):
        """CSA ratio-4 selection producer. index_query [B, S, H, 128] f32,
        index_weight [B, S, H] f32, index_keys [B, key_cap, 68] u8, total_len
        int64 device tensor of one element, selected [B, out_heads, S, K] i32
        (written), workspace a device tensor of csa_index_workspace_bytes bytes."""
        B, S, H, _ = index_query.shape
        self._sync_stream()
        self._check(self.lib.sparse_attn_csa_index_select(
            self.handle, _ptr(index_query), _ptr(index_weight), _ptr(index_keys), B, S, H,
            index_keys.shape[1], _ptr(total_len), selected.shape[3], selected.shape[1], _ptr(selected),
            _ptr(workspace)))

    def reset_error_async(self):
        self._sync_stream()
        self._check(self.lib.sparse_attn_reset_error_async(self.handle))

    def read_error(self, raise_on_error=False):
        """Synchronise and return (word, first_bad, message)."""
        self._sync_stream()
        w, fb = ctypes.c_uint32(), ctypes.c_uint64()
        st = self.lib.sparse_attn_read_error(self.handle, ctypes.byref(w), ctypes.byref(fb))
        msg = self.last_error()
        if st not in (SA_OK, SA_E_INDEX):
            raise SparseAttnError(st, msg)
        if raise_on_error and st == SA_E_INDEX:
            raise SparseAttnError(st, msg)
        return int(w.value), int(fb.value), msg

    def profile_enable(self, max_launches):
        self._sync_stream()
        self._check(self.lib.sparse_attn_profile_enable(self.handle, max_launches))

    def profile_read(self):
        """(summed ms, launches) of the main forward kernel since the last read."""
        self._sync_stream()
        ms, n = ctypes.c_double(), ctypes.c_int64()
        self._check(self.lib.sparse_attn_profile_read(self.handle, ctypes.byref(ms), ctypes.byref(n)))
        return float(ms.value), int(n.value)

    def measure_copy(self, dst, src, nbytes):
        """Streaming device copy of nbytes (peak probe; HBM traffic 2 * nbytes)."""
        self._sync_stream()
        self._check(self.lib.sparse_attn_measure_copy(self.handle, _ptr(dst), _ptr(src), nbytes))

    def measure_read(self, sink, src, nbytes):
        """Streaming device read of nbytes (peak probe); sink: uint32 [SA_PEAK_READ_SINK_WORDS]."""
        self._sync_stream()
        self._check(self.lib.sparse_attn_measure_read(self.handle, _ptr(sink), _ptr(src), nbytes))

    def measure_mfma(self, out, workgroups, iters):
        """bf16 matrix-core loop (peak probe): workgroups * 4 * iters * 8 * 16384 flops."""
        self._sync_stream()
        self._check(self.lib.sparse_attn_measure_mfma(self.handle, _ptr(out), workgroups, iters))

    def query_plan(self, batch, q_seq, index_heads, width):
        p, s = ctypes.c_int32(), ctypes.c_int32()
        self._check(self.lib.sparse_attn_query_plan(self.handle, batch, q_seq, index_heads, width,
                                                    ctypes.byref(p), ctypes.byref(s)))
        return int(p.value), int(s.value)


def forward_latent_static(q, batch, q_seq, cache, cache_capacity, valid_len, indices, width, y, *,
                          index_dtype=SA_IDX_I32, scale=0.0, softcap=0.0, stream=None):
    """sparse_attn_forward_latent_static on the current (or given) torch stream:
    the shared-latent bf16 forward without a context, its split-K partials in
    the library's static per-GPU scratch."""
    lib = load()
    st = lib.sparse_attn_forward_latent_static(
        _ptr(q), batch, q_seq, _ptr(cache), cache_capacity, _ptr(valid_len), _ptr(indices),
        index_dtype, width, scale, softcap, _ptr(y), _stream_handle(stream))
    if st != SA_OK:
        raise SparseAttnError(st, lib.sparse_attn_last_error(None).decode())


def __getattr__(name):
    # module-level access to the raw C entry points under their own names
    if name in EXPORTS:
        return getattr(load(), name)
    raise AttributeError(name)
