"""The allocation-free shared-latent forward against sparse_attn_forward.

sparse_attn_forward_latent_static runs the same kernels as sparse_attn_forward
(fused_validate = 0) on a shared-latent bf16 context, with its split-K
partials in the library's static per-GPU scratch instead of the context's
buffers. Two calls in a row, the second smaller (and with a ragged index
width and per-batch lengths), must each equal the context call bit for bit.
"""
import numpy as np
import pytest

import sparse_attention_kv_append_amd as sa

pytestmark = pytest.mark.gpu

NH, DK, DV = 64, 576, 512


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


def bf16_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def make_inputs(seed, batch, cap, width, valid):
    rng = np.random.default_rng(seed)
    q = bf16_bits(rng, (batch, NH, 1, DK))
    cache = bf16_bits(rng, (batch, 1, cap, DK), 0.5)
    idx = np.full((batch, 1, 1, width), -1, dtype=np.int32)
    for b in range(batch):
        n = int(rng.integers(1, min(width, valid[b]) + 1))
        idx[b, 0, 0, :n] = np.sort(rng.choice(valid[b], size=n, replace=False))
    return q, cache, idx


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def run_pair(seed, batch, cap, width, idx64=False):
    import torch
    valid = np.random.default_rng(seed + 1).integers(width // 2, cap + 1, size=batch).astype(np.int32)
    q, cache, idx = make_inputs(seed, batch, cap, width, valid)
    if idx64:
        idx = idx.astype(np.int64)
    dq, dc, di, dv = dev(q), dev(cache), dev(idx), dev(valid)
    ctx = sa.Context(num_heads=NH, kv_num_heads=1, head_dim_qk=DK, head_dim_v=DV, dtype=sa.SA_BF16,
                     kv_layout=sa.SA_KV_SHARED_LATENT, index_dtype=sa.SA_IDX_I64 if idx64 else sa.SA_IDX_I32,
                     max_batch=batch, max_q_seq=1, max_index_width=width, max_cache_len=cap)
    path, splits = ctx.query_plan(batch, 1, 1, width)
    assert path == 2
    banner(f"static forward: batch {batch} cap {cap} width {width} idx64 {idx64} splits {splits}")
    y_ref = torch.full((batch, NH, 1, DV), float("nan"), dtype=torch.bfloat16, device="cuda")
    ctx.forward(dq, batch, 1, dc, None, cap, dv, di, 1, width, y_ref, fused_validate=False)
    y = torch.full_like(y_ref, float("nan"))
    sa.forward_latent_static(dq, batch, 1, dc, cap, dv, di, width, y,
                             index_dtype=sa.SA_IDX_I64 if idx64 else sa.SA_IDX_I32)
    torch.cuda.synchronize()
    ctx.destroy()
    a = y_ref.view(torch.int16).cpu().numpy()
    b = y.view(torch.int16).cpu().numpy()
    assert not np.isnan(y.float().cpu().numpy()).any()
    assert np.array_equal(a, b), f"{(a != b).sum()} of {a.size} outputs differ"
    return splits


def test_static_forward_matches_the_context_forward_on_two_calls():
    # the decode shape (8 splits, 256 partials), then a smaller ragged call that
    # reuses the scratch the first one left behind
    assert run_pair(11, 32, 4096, 2048) > 1
    assert run_pair(12, 5, 1500, 700, idx64=True) > 1


def test_static_forward_single_split_and_capacity_error():
    import torch
    # enough rows to fill the chip without splitting: no scratch is used
    assert run_pair(13, 260, 300, 96) == 1
    p = torch.empty(8, device="cuda")
    with pytest.raises(sa.SparseAttnError) as e:
        sa.forward_latent_static(p, 200, 1, p, 8192, None, p, 4096, p)
    assert e.value.status == sa.SA_E_CAPACITY
