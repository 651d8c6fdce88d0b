"""GPU index validation against the oracle, bit for bit: per-row classes, the
error word and the first failing (row, column), plus the message the library
builds for it (the IndexShare host validator's wording)."""
import numpy as np
import pytest

import oracle
from gpu_support import tt

pytestmark = pytest.mark.gpu


def plant(rng, B, Hi, Sq, W, bound):
    """Valid rows with one planted violation class in most of them."""
    idx = np.full((B, Hi, Sq, W), -1, np.int64)
    rows = idx.reshape(-1, W)
    for r in range(rows.shape[0]):
        T = int(bound[r // (Hi * Sq)])
        n = int(rng.integers(1, min(W, T) + 1))
        rows[r, :n] = np.sort(rng.choice(T, size=n, replace=False))
        kind = rng.integers(0, 8)
        c = int(rng.integers(0, W))
        if kind == 1:
            rows[r, c] = -int(rng.integers(2, 9))                # sentinel
        elif kind == 2 and n < W:
            rows[r, int(rng.integers(n, W))] = int(rng.integers(0, T))  # after padding
        elif kind == 3:
            rows[r, min(c, n - 1)] = T + int(rng.integers(0, 5))  # range
        elif kind == 4 and n >= 2:
            j = int(rng.integers(1, n))
            rows[r, j] = rows[r, j - 1]                            # duplicate
        elif kind == 5 and n >= 2:
            j = int(rng.integers(1, n))
            rows[r, j - 1], rows[r, j] = rows[r, j], rows[r, j - 1]  # order
        elif kind == 6:
            rows[r, :] = -1                                          # all padding
    return idx


@pytest.mark.parametrize("W", [1, 3, 63, 64, 65, 130, 2048])
@pytest.mark.parametrize("i64", [False, True])
def test_validation_matches_oracle(W, i64):
    import torch
    import sparse_attention_kv_append_amd as sa
    print(f"\n[gpu] validate W={W} i64={i64}", flush=True)
    rng = np.random.default_rng(W * 7 + i64)
    B, Hi, Sq = 3, 2, 5
    bound = np.array([W + 3, 2 * W + 1, max(1, W // 2)], np.int32)
    idx = plant(rng, B, Hi, Sq, W, bound)
    if not i64:
        idx = idx.astype(np.int32)
    word, cls, first, msg = oracle.validate_indices(idx, bound)
    ctx = sa.Context(num_heads=Hi, kv_num_heads=1, head_dim_qk=64, head_dim_v=64, dtype=sa.SA_BF16,
                     index_dtype=sa.SA_IDX_I64 if i64 else sa.SA_IDX_I32, max_batch=B,
                     max_q_seq=Sq, max_index_width=W, max_cache_len=4096)
    row_class = torch.zeros(B * Hi * Sq, dtype=torch.uint8, device="cuda")
    ctx.reset_error_async()
    ctx.validate_indices(tt(idx), B, Hi, Sq, W, valid_len=tt(bound), row_class=row_class)
    dword, dfirst, dmsg = ctx.read_error()
    assert np.array_equal(row_class.cpu().numpy(), cls)
    assert dword == word
    if first is None:
        assert dfirst == 2 ** 64 - 1 and dmsg == ""
    else:
        assert dfirst == first[0] * (W + 1) + first[1]
        assert dmsg == msg
    ctx.destroy()


def test_words_accumulate_until_reset_and_external_word():
    import torch
    import sparse_attention_kv_append_amd as sa
    ctx = sa.Context(num_heads=1, kv_num_heads=1, head_dim_qk=64, head_dim_v=64, dtype=sa.SA_BF16,
                     max_batch=1, max_q_seq=1, max_index_width=4, max_cache_len=16)
    bad = tt(np.array([[[[0, 0, -1, -1]]]], np.int32))
    good = tt(np.array([[[[0, 1, -1, -1]]]], np.int32))
    ctx.reset_error_async()
    ctx.validate_indices(bad, 1, 1, 1, 4, cache_len=16)
    ctx.validate_indices(good, 1, 1, 1, 4, cache_len=16)
    w, _, msg = ctx.read_error()
    assert w == (sa.SA_ERR_DUPLICATE | sa.SA_ERR_INDEX_ANY)
    assert msg.endswith("column=1]: duplicate index 0")
    ctx.reset_error_async()
    assert ctx.read_error()[0] == 0
    ext = torch.zeros(1, dtype=torch.int32, device="cuda")
    fb = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    ctx.validate_indices(tt(np.array([[[[-3, -1, -1, -1]]]], np.int32)), 1, 1, 1, 4, cache_len=16,
                         error_word=ext, first_bad=fb)
    torch.cuda.synchronize()
    assert int(ext.item()) == (sa.SA_ERR_SENTINEL | sa.SA_ERR_INDEX_ANY)
    assert int(fb.item()) == 0
    assert ctx.read_error()[0] == 0  # the context word was not touched
    ctx.destroy()
