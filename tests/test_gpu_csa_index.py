"""GPU parity of the CSA selection producer (sparse_attn_csa_index_select,
through the C ABI) against the oracle on the same seeded inputs.

The selection is integer output decided by fp32 scores, and both sides take
every step in the same fp32 operations (the RoPE's pow, sin and cos exactly
rounded on both), so the bar is bit-exact: the device's rows equal the
oracle's, and its scores (read from the workspace) equal the oracle's scores.
Each row is also checked to be a valid top-k of the oracle's scores (distinct
complete records, -1 padded, non-increasing, the cut at k), which names the
row if the equality ever fails.
"""
import numpy as np
import pytest

import oracle
import sa_workloads as W

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


def sa_mod():
    import sparse_attention_kv_append_amd as sa
    return sa


@pytest.fixture(scope="module")
def ctx():
    import sparse_attention_kv_append_amd as sa
    return sa.Context(num_heads=16, kv_num_heads=1, head_dim_qk=64, head_dim_v=64, dtype=sa.SA_F32)


def run_gpu(ctx, inp, total, K, out_heads):
    import torch
    dev = "cuda"
    iq = torch.from_numpy(inp["index_query"]).to(dev)
    iw = torch.from_numpy(inp["index_weight"]).to(dev)
    keys = torch.from_numpy(np.ascontiguousarray(inp["index_keys"])).to(dev)
    B, S, H, _ = iq.shape
    tot = torch.tensor([total], dtype=torch.int64, device=dev)
    sel = torch.full((B, out_heads, S, K), -7, dtype=torch.int32, device=dev)
    kcap = keys.shape[1]
    ws = torch.empty(ctx.csa_index_workspace_bytes(B, S, H, kcap), dtype=torch.uint8, device=dev)
    ctx.reset_error_async()
    ctx.csa_index_select(iq, iw, keys, tot, sel, ws)
    torch.cuda.synchronize()
    word, _, msg = ctx.read_error()
    # the workspace starts with the scores, fp32 [B, S, key_cap]
    scores = ws[:B * S * kcap * 4].cpu().numpy().view(np.float32).reshape(B, S, kcap)
    return sel.cpu().numpy(), word, msg, scores


def check_selection(gsel, osel, scores, total, key_cap, rtol=1e-5):
    """gsel [B, S, K] device rows vs the oracle's rows and scores; returns the
    number of rows equal to the oracle's."""
    B, S, K = gsel.shape
    same = 0
    for b in range(B):
        for s in range(S):
            pos = total - S + s
            n = min((pos + 1) // 4, key_cap)
            g = gsel[b, s]
            k = min(K, n)
            assert (g[k:] == -1).all(), (b, s)
            top = g[:k]
            assert len(set(top.tolist())) == k and (top >= 0).all() and (top < n).all(), (b, s)
            sc = scores[b, s, :n].astype(np.float64)
            tol = rtol * max(1.0, np.abs(sc).max())
            gs = sc[top]
            assert (np.diff(gs) <= tol).all(), (b, s)                      # non-increasing
            rest = np.setdiff1d(np.arange(n), top)
            if len(rest):
                assert gs.min() >= sc[rest].max() - tol, (b, s)            # the cut at k
            same += int(np.array_equal(g, osel[b, s]))
    return same


@pytest.mark.parametrize("kw", [
    dict(),                                                     # S 3, H 16, 300 keys, K 40, 2 out heads
    dict(heads=64, key_cap=1500, total=5000, topk=512),         # several score workgroups, K 512
    dict(heads=48, seq=4, key_cap=2100, total=8403, topk=2048), # K 2048 > complete records: padding
    dict(batch=1, seq=7, heads=32, key_cap=40, total=150, topk=64),  # causal domain grows per query
])
def test_index_select_matches_oracle(ctx, kw):
    w = W.CSA_INDEX_WORKLOADS["csa_index_small"].scaled(**kw)
    inp = W.make_csa_index_numpy(w)
    banner(f"csa index {w}")
    osel, flags, scores = oracle.csa_index_select(inp["index_query"], inp["index_weight"], inp["index_keys"],
                                                  w.total, w.topk, with_scores=True)
    assert flags == 0
    gsel, word, msg, gscores = run_gpu(ctx, inp, w.total, w.topk, w.out_heads)
    assert word == 0, msg
    for h in range(1, w.out_heads):
        np.testing.assert_array_equal(gsel[:, h], gsel[:, 0])
    same = check_selection(gsel[:, 0], osel, scores, w.total, w.key_cap)
    for b in range(w.batch):
        for s in range(w.seq):
            n = min((w.total - w.seq + s + 1) // 4, w.key_cap)
            np.testing.assert_array_equal(gscores[b, s, :n], scores[b, s, :n])
    assert same == w.batch * w.seq


def run_and_compare(ctx, w, inp):
    osel, flags, scores = oracle.csa_index_select(inp["index_query"], inp["index_weight"], inp["index_keys"],
                                                  w.total, w.topk, with_scores=True)
    gsel, word, msg, gscores = run_gpu(ctx, inp, w.total, w.topk, w.out_heads)
    # exact ties (many keys of one dominant block score 0 over every head) are
    # ordered by ascending record on both sides, and reported by both
    assert (flags & ~oracle.SEL_TIE) == 0, flags
    assert word == (sa_mod().SA_ERR_INDEX_TIE if flags & oracle.SEL_TIE else 0), (flags, word, msg)
    for b in range(w.batch):
        for s in range(w.seq):
            n = min((w.total - w.seq + s + 1) // 4, w.key_cap)
            np.testing.assert_array_equal(gscores[b, s, :n], scores[b, s, :n], err_msg=f"scores of row {(b, s)}")
            np.testing.assert_array_equal(gsel[b, 0, s], osel[b, s], err_msg=f"selection of row {(b, s)}")


@pytest.mark.parametrize("kw", [dict(), dict(heads=64, key_cap=1500, total=5000, topk=512)])
def test_index_select_on_keys_of_uneven_blocks_quantized_by_the_oracle(ctx, kw):
    """Keys from the oracle's own FP4 quantizer on data whose 32-dim blocks
    differ in magnitude by up to 2^24: their scale bytes spread far beyond a
    range where the matrix dot is exact, so the ordered fold decides."""
    w = W.CSA_INDEX_WORKLOADS["csa_index_small"].scaled(**kw)
    inp = W.make_csa_index_numpy(w)
    rng = np.random.default_rng(77)
    raw = rng.standard_normal((w.batch, w.key_cap, 128)).astype(np.float32)
    raw *= np.repeat(np.exp2(rng.integers(-12, 13, (w.batch, w.key_cap, 4))).astype(np.float32), 32, axis=-1)
    inp["index_keys"] = oracle.fp4_pack_keys(raw)
    sb = inp["index_keys"][:, :, 0::17].astype(int)
    assert (sb.max(-1) - sb.min(-1)).max() >= 16  # blocks of one key far apart
    banner(f"csa index, oracle-quantized uneven keys {w}")
    run_and_compare(ctx, w, inp)


def test_index_select_on_planted_wide_scale_bytes(ctx):
    """Random codes with block scale bytes planted over 0..200 within one key
    (subnormal and zero-exponent key values among them): bit-exact scores
    and selection."""
    w = W.CSA_INDEX_WORKLOADS["csa_index_small"].scaled(heads=32, key_cap=700, total=2400, topk=96)
    inp = W.make_csa_index_numpy(w)
    rng = np.random.default_rng(78)
    keys = inp["index_keys"]
    keys[:, :, 0::17] = rng.integers(90, 170, keys[:, :, 0::17].shape, dtype=np.uint8)
    keys[:, ::7, 0] = 0                        # 2^-127: subnormal key values
    keys[:, 3::11, 17] = rng.integers(1, 12, keys[:, 3::11, 17].shape, dtype=np.uint8)
    keys[:, 5::13, 51] = 200
    banner(f"csa index, planted wide scale bytes {w}")
    run_and_compare(ctx, w, inp)


def test_index_select_geometry_and_nonfinite(ctx):
    import sparse_attention_kv_append_amd as sa
    w = W.CSA_INDEX_WORKLOADS["csa_index_small"]
    inp = W.make_csa_index_numpy(w)
    _, word, _, _ = run_gpu(ctx, inp, 2, w.topk, 1)  # total 2 < S 3
    assert word == sa.SA_ERR_CSA_GEOMETRY
    inp["index_weight"][1, 2, 5] = np.inf
    _, flags = oracle.csa_index_select(inp["index_query"], inp["index_weight"], inp["index_keys"], w.total, w.topk)
    assert flags & oracle.SEL_NONFINITE
    _, word, _, _ = run_gpu(ctx, inp, w.total, w.topk, 1)
    # an infinite weight makes many scores +inf: equal, so both sides report a tie too
    assert word == sa.SA_ERR_INDEX_NONFINITE | (sa.SA_ERR_INDEX_TIE if flags & oracle.SEL_TIE else 0)


def test_index_select_host_errors(ctx):
    import torch

    import sparse_attention_kv_append_amd as sa
    dev = "cuda"
    iq = torch.zeros((1, 1, 24, 128), device=dev)
    iw = torch.zeros((1, 1, 24), device=dev)
    keys = torch.zeros((1, 8, 68), dtype=torch.uint8, device=dev)
    tot = torch.tensor([8], dtype=torch.int64, device=dev)
    sel = torch.zeros((1, 1, 1, 4), dtype=torch.int32, device=dev)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    with pytest.raises(sa.SparseAttnError) as e:
        ctx.csa_index_select(iq, iw, keys, tot, sel, ws)  # 24 heads
    assert e.value.status == sa.SA_E_UNSUPPORTED


def test_index_select_fullsize_sampled_rows():
    """The benchmark's workload (batch 64, 64 index heads, 16384 keys, top-512)
    in its launch configuration; sampled rows against the oracle on those rows."""
    import torch

    import bench
    banner("csa index full size: building inputs")
    s = bench.CsaIndexSetup("csa_index_decode", 1)
    s.step(0)
    torch.cuda.synchronize()
    word, _, msg = s.ctx.read_error()
    # among 16384 fp32 scores per row an exactly equal pair is a likely
    # birthday collision: the device may report one (for any row)
    assert word & ~sa_mod().SA_ERR_INDEX_TIE == 0, msg
    gsel = s.sel.cpu().numpy()[:, 0]
    bs = [0, 9, 33, 63]
    same = 0
    for b in bs:
        banner(f"csa index full size: oracle on batch entry {b}")
        inp = s.oracle_inputs(b)
        osel, flags, scores = oracle.csa_index_select(inp["index_query"], inp["index_weight"], inp["index_keys"],
                                                      s.w.total, s.w.topk, with_scores=True)
        # both sides order equal scores by ascending record; a tie the oracle
        # sees in a sampled row the device must have reported
        assert flags & ~oracle.SEL_TIE == 0
        if flags & oracle.SEL_TIE:
            assert word & sa_mod().SA_ERR_INDEX_TIE
        same += check_selection(gsel[b:b + 1], osel, scores, s.w.total, s.w.key_cap)
    assert same == len(bs)
    s.ctx.destroy()


def test_index_select_ties_at_the_cut(ctx):
    """Identical keys give identical scores: every cut falls inside a tie, and
    both sides take the tied records in ascending record order."""
    w = W.CSA_INDEX_WORKLOADS["csa_index_small"]
    inp = W.make_csa_index_numpy(w)
    inp["index_keys"][:, 100:220] = inp["index_keys"][:, 7:8]   # 120 copies of record 7
    inp["index_keys"][1, :] = inp["index_keys"][1, 3:4]         # batch entry 1: all identical
    osel, flags, scores = oracle.csa_index_select(inp["index_query"], inp["index_weight"], inp["index_keys"],
                                                  w.total, w.topk, with_scores=True)
    assert flags & oracle.SEL_TIE
    gsel, word, msg, gscores = run_gpu(ctx, inp, w.total, w.topk, w.out_heads)
    assert word == sa_mod().SA_ERR_INDEX_TIE, msg   # reported, as the CPU page would refuse the rows
    np.testing.assert_array_equal(gsel[:, 0], osel)
    np.testing.assert_array_equal(gsel[1, 0, :, :w.topk], np.broadcast_to(np.arange(w.topk), (w.seq, w.topk)))
