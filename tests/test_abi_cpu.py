"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/sparse_attn.h declares, and refuses bad configurations
and NULL / unknown contexts with the documented status before launching."""
import ctypes
import re
from pathlib import Path

import pytest

import sparse_attention_kv_append_amd as sa

HEADER = Path(__file__).resolve().parent.parent / "include" / "sparse_attn.h"


def declared_functions():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\**(sparse_attn_[a-z_]+)\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = sa.load()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(sa.EXPORTS)
    assert lib.sparse_attn_version().decode().startswith("sparse_attn")


def test_struct_layout_matches_header():
    # 9 int32 + 2 float + 4 int64, naturally aligned: 44 bytes padded to 48, + 32
    assert ctypes.sizeof(sa.sa_config) == 80


def _cfg(**kw):
    base = dict(num_heads=4, kv_num_heads=2, head_dim_qk=64, head_dim_v=64, rope_dim=0,
                dtype=sa.SA_BF16, cache_format=sa.SA_CACHE_DENSE, kv_layout=sa.SA_KV_SEPARATE,
                index_dtype=sa.SA_IDX_I32, scale=0.0, softcap=0.0, max_batch=1, max_q_seq=1,
                max_index_width=8, max_cache_len=8)
    base.update(kw)
    return sa.sa_config(*[base[f] for f, _ in sa.sa_config._fields_])


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=0), sa.SA_E_ARG),
    (dict(num_heads=6, kv_num_heads=4), sa.SA_E_ARG),
    (dict(dtype=7), sa.SA_E_DTYPE),
    (dict(head_dim_v=32), sa.SA_E_SHAPE),                        # separate needs Dv == Dk
    (dict(kv_layout=sa.SA_KV_SHARED_LATENT, head_dim_v=96), sa.SA_E_SHAPE),
    (dict(cache_format=sa.SA_CACHE_FP8_E4M3_BLOCK64), sa.SA_E_DTYPE),  # fp8 needs shared latent
    (dict(cache_format=sa.SA_CACHE_FP8_E4M3_BLOCK64, kv_layout=sa.SA_KV_SHARED_LATENT,
          head_dim_qk=100, head_dim_v=64, rope_dim=4), sa.SA_E_SHAPE),
    (dict(scale=float("nan")), sa.SA_E_ARG),
    (dict(scale=-1.0), sa.SA_E_ARG),
    (dict(softcap=float("inf")), sa.SA_E_ARG),
    (dict(max_batch=0), sa.SA_E_ARG),
    (dict(index_dtype=3), sa.SA_E_DTYPE),
    (dict(head_dim_qk=1024, head_dim_v=1024), sa.SA_E_UNSUPPORTED),
])
def test_create_rejects_bad_config(kw, status):
    lib = sa.load()
    h = ctypes.c_void_p()
    cfg = _cfg(**kw)
    assert lib.sparse_attn_create(ctypes.byref(cfg), None, ctypes.byref(h)) == status
    assert h.value is None


def test_null_and_unknown_context_rejected_without_launch():
    lib = sa.load()
    assert lib.sparse_attn_forward(None, None, 1, 1, None, None, 1, None, None, 1, 1, None, 0) == sa.SA_E_STATE
    assert lib.sparse_attn_kv_append(None, 1, None, None, 0, None, None, None, 1, 0, None, None, 1,
                                     None) == sa.SA_E_STATE
    assert lib.sparse_attn_validate_indices(None, None, 1, 1, 1, 1, None, 1, None, None, None) == sa.SA_E_STATE
    assert lib.sparse_attn_reset_error_async(None) == sa.SA_E_STATE
    assert lib.sparse_attn_csa_forward(None, None, 1, 1, 16, None, 1, None, 1, None, 1, 1, None, None, None,
                                       None, 0.0, None) == sa.SA_E_STATE
    assert lib.sparse_attn_forward_bias(None, None, 1, 1, None, None, 1, None, None, 1, 1, None, None, 0,
                                        None, 0) == sa.SA_E_STATE
    assert lib.sparse_attn_capacity_lengths(None, None, None, 0, 1, 1, 1, 1, None, None) == sa.SA_E_STATE
    assert lib.sparse_attn_capacity_step(None, None, 1, 1, None, None, 1, None, None, 1, None, 1, 1, None, None, 0,
                                         None, None, None, 1) == sa.SA_E_STATE
    fake = ctypes.c_void_p(0x1234)
    assert lib.sparse_attn_capacity_lengths(fake, None, None, 0, 1, 1, 1, 1, None, None) == sa.SA_E_STATE
    assert lib.sparse_attn_forward(fake, None, 1, 1, None, None, 1, None, None, 1, 1, None, 0) == sa.SA_E_STATE
    assert lib.sparse_attn_destroy(None) == sa.SA_OK
    assert b"invalid" in lib.sparse_attn_last_error(fake)


def test_static_forward_checks_arguments_before_any_hip_call():
    """The allocation-free forward rejects bad arguments and a split-K plan
    whose partials exceed its static scratch on the host, before touching the
    device (so this runs without a GPU)."""
    lib = sa.load()
    p = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails before a launch
    f = lib.sparse_attn_forward_latent_static
    assert f(None, 1, 1, p, 64, None, p, sa.SA_IDX_I32, 64, 0.0, 0.0, p, None) == sa.SA_E_ARG
    assert b"required" in lib.sparse_attn_last_error(None)
    assert f(p, 0, 1, p, 64, None, p, sa.SA_IDX_I32, 64, 0.0, 0.0, p, None) == sa.SA_E_ARG
    assert f(p, 1, 1, p, 64, None, p, 7, 64, 0.0, 0.0, p, None) == sa.SA_E_DTYPE
    assert f(p, 1, 1, p, 64, None, p, sa.SA_IDX_I32, 64, -1.0, 0.0, p, None) == sa.SA_E_ARG
    assert f(p, 1, 1, p, 64, None, p, sa.SA_IDX_I32, 64, 0.0, float("nan"), p, None) == sa.SA_E_ARG
    # 200 rows of 4096 columns plan 2 splits: 400 partials of 131,584 bytes > 48 MiB
    assert f(p, 200, 1, p, 8192, None, p, sa.SA_IDX_I32, 4096, 0.0, 0.0, p, None) == sa.SA_E_CAPACITY
    msg = lib.sparse_attn_last_error(None)
    assert b"static scratch holds 50331648" in msg and b"52633600" in msg, msg
    assert sa.SA_STATIC_SCRATCH_BYTES == 48 << 20
