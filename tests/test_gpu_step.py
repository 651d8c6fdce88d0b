"""sparse_attn_step (reset + in-place append + forward with fused validation
in one call) against the same three calls made separately, and against the
oracle.

On the bf16 shared-latent path with at most 8 current rows the step is one
forward launch in which every workgroup writes its batch's new rows itself;
the index rows below always select the newest row, so workgroups read rows
they have just written. Y, the cache bytes, present_len and the error word
must equal those of the separate calls bit for bit (same kernel arithmetic),
including the reset semantics and a capacity failure."""
import numpy as np
import pytest

import oracle
import sa_workloads as W
from gpu_support import check_close, make_ctx, oracle_records, tt

pytestmark = pytest.mark.gpu

DEC = W.WORKLOADS["decode_bf16"]
FP8 = W.WORKLOADS["decode_fp8"]
CASES = {
    "decode_split": DEC.scaled(batch=6, past=1500, topk=700, width=710, capacity=1600),
    "multi_row": DEC.scaled(batch=2, q_seq=4, cur=4, past=300, topk=200, width=210, capacity=320),
    "eight_rows": DEC.scaled(batch=3, q_seq=8, cur=8, past=260, topk=100, width=100, capacity=300),
    "long_cur": DEC.scaled(batch=2, q_seq=12, cur=12, past=300, topk=200, width=210, capacity=330),
    "fp8_split": FP8.scaled(batch=6, past=1200, topk=650, width=650, capacity=1300),
    "fp8_multi_row": FP8.scaled(batch=2, q_seq=3, cur=3, past=400, topk=300, width=300, capacity=420),
    # 260 rows: one workgroup per row, which records its own row's verdict and
    # counts toward the launch's record in the same launch as the append
    "one_split_rows": DEC.scaled(batch=130, q_seq=2, cur=2, past=200, topk=100, width=110, capacity=240),
    "fp8_one_split_rows": FP8.scaled(batch=130, q_seq=2, cur=2, past=200, topk=100, width=110, capacity=240),
}
# fp8 current rows as packed records (byte append) or as bf16 rows quantized on the device
QUANT = {"fp8_split": [False, True], "fp8_multi_row": [True], "fp8_one_split_rows": [True]}


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


def with_newest(idx, total):
    """Every row's last selected key becomes the newest row (total - 1)."""
    out = idx.copy()
    for row in out.reshape(-1, out.shape[-1]):
        n = int((row >= 0).sum())
        if n and total - 1 not in row[:n]:
            row[n - 1] = total - 1
    return out


def setup(w, seed=0):
    import torch
    inp = W.make_numpy(w)
    idx = with_newest(inp["indices"], w.total)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    if w.cache_format == W.CACHE_FP8:
        recs = oracle_records(inp["past_k"][:, :, :w.past], w)
        cache = torch.randint(0, 120, (w.batch, 1, w.cap, recs.shape[-1]), dtype=torch.uint8, device="cuda",
                              generator=gen)
        cache[:, :, :w.past] = tt(recs)
        return inp, idx, cache
    garbage = torch.randint(-30000, 30000, (w.batch, 1, w.cap, w.dk), dtype=torch.int16, device="cuda",
                            generator=gen)
    cache = garbage.clone()
    cache[:, :, :w.past] = tt(inp["past_k"][:, :, :w.past]).view(torch.int16)
    return inp, idx, cache


def cur_rows(w, inp, quant):
    """Current rows as passed: bf16 rows (bf16 caches, or fp8 to quantize) or records."""
    if w.cache_format == W.CACHE_FP8 and not quant:
        return tt(oracle_records(inp["cur_k"], w))
    return tt(inp["cur_k"])


def run_separate(ctx, w, inp, idx, cache, reset=True, quant=False):
    import torch
    B = w.batch
    plen = tt(inp["past_len"])
    prl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    y = torch.full((B, w.hq, w.q_seq, w.dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    if reset:
        ctx.reset_error_async()
    ctx.kv_append(B, cache, None, w.cap, plen, cur_rows(w, inp, quant), None, w.cur, cache, None, w.cap,
                  present_len=prl, cur_is_unquantized_bf16=quant)
    ctx.forward(tt(inp["q"]), B, w.q_seq, cache, None, w.cap, prl, tt(idx), 1, w.width, y,
                fused_validate=True)
    word, fb, msg = ctx.read_error()
    return y, prl, word, fb, msg


def run_step(ctx, w, inp, idx, cache, reset=True, quant=False):
    import torch
    B = w.batch
    plen = tt(inp["past_len"])
    prl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    y = torch.full((B, w.hq, w.q_seq, w.dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    ctx.step(tt(inp["q"]), B, w.q_seq, cache, w.cap, plen, cur_rows(w, inp, quant), w.cur, prl, tt(idx), 1,
             w.width, y, reset_error=reset, cur_is_unquantized_bf16=quant)
    word, fb, msg = ctx.read_error()
    return y, prl, word, fb, msg


STEP_CASES = [(n, qz) for n in CASES for qz in QUANT.get(n, [False])]


@pytest.mark.parametrize("name,quant", STEP_CASES)
def test_step_matches_separate_calls(name, quant):
    import torch
    w = CASES[name]
    banner(f"step {name} quant={quant}")
    inp, idx, cache = setup(w)
    ctx = make_ctx(w)
    c1, c2 = cache.clone(), cache.clone()
    ya, pa, wa, _, ma = run_separate(ctx, w, inp, idx, c1, quant=quant)
    yb, pb, wb, _, mb = run_step(ctx, w, inp, idx, c2, quant=quant)
    assert wa == 0 and wb == 0, (ma, mb)
    assert torch.equal(pa, pb) and torch.equal(pb, tt(inp["valid_len"]))
    assert torch.equal(c1, c2)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    # and the oracle
    if w.cache_format == W.CACHE_FP8:
        pk = oracle.kv_append(oracle_records(inp["past_k"], w), inp["past_len"], oracle_records(inp["cur_k"], w))
        assert np.array_equal(c2[:, :, :w.total].cpu().numpy(), pk[:, :, :w.total])
        fmt = oracle.FP8_BLOCK64
    else:
        pk = oracle.kv_append(inp["past_k"].copy(), inp["past_len"], inp["cur_k"])
        fmt = w.dtype
    ref = oracle.forward(inp["q"], pk, None, idx, q_dtype=w.dtype, cache_fmt=fmt, kv_layout=w.layout,
                         hkv=w.hkv, dv=w.dv, rope=w.rope, scale=w.scale, softcap=w.softcap, threads=8)
    check_close(yb.float().cpu().numpy(), ref, w.dtype, name)
    ctx.destroy()


def test_step_fp8_nonfinite_row_left_unwritten():
    """A current bf16 row holding an infinity: nothing is written for it and
    the word says so, in one launch as in the separate calls."""
    import torch
    w = CASES["fp8_split"]
    banner("step fp8 non-finite row")
    inp, idx, cache = setup(w)
    inp = dict(inp)
    inp["cur_k"] = inp["cur_k"].copy()
    inp["cur_k"][4, 0, 0, 77] = 0x7f80  # +inf in batch 4's current row
    ctx = make_ctx(w)
    c1, c2 = cache.clone(), cache.clone()
    _, _, wa, _, _ = run_separate(ctx, w, inp, idx, c1, quant=True)
    _, _, wb, _, _ = run_step(ctx, w, inp, idx, c2, quant=True)
    want = sa_bits("QUANT_NONFINITE") | sa_bits("APPEND_ANY")
    assert wa & want == want and wb & want == want
    assert torch.equal(c1, c2) and torch.equal(c2[4, :, w.past], cache[4, :, w.past])
    ctx.destroy()


def bad_rows(idx):
    out = idx.copy()
    out[0, 0, 0, 3] = out[0, 0, 0, 2]  # a duplicate in row 0
    return out


@pytest.mark.parametrize("name", ["decode_split", "long_cur", "one_split_rows", "fp8_one_split_rows"])
def test_step_reset_semantics(name):
    """Without reset the step adds its bits to an earlier launch's; with reset
    it replaces them (word, first failing position and message)."""
    w = CASES[name]
    banner(f"step reset semantics {name}")
    inp, idx, cache = setup(w)
    ctx = make_ctx(w)
    bad = bad_rows(idx)
    # an earlier failing validation latches ORDER in a row of the last batch
    early = idx.copy()
    r = early[-1, 0, -1]
    r[1], r[2] = r[2], r[1]
    vl = tt(inp["valid_len"])

    def latch_early():
        ctx.reset_error_async()
        ctx.validate_indices(tt(early), w.batch, 1, w.q_seq, w.width, valid_len=vl)
        return ctx.read_error()

    e_word, e_fb, e_msg = latch_early()
    assert e_word == (sa_bits("ORDER") | 512)
    _, _, w0, fb0, m0 = run_step(ctx, w, inp, idx, cache.clone(), reset=False)
    assert (w0, fb0, m0) == (e_word, e_fb, e_msg)          # kept
    latch_early()
    _, _, w1, fb1, _ = run_step(ctx, w, inp, idx, cache.clone(), reset=True)
    assert w1 == 0 and fb1 == 2 ** 64 - 1                  # replaced by a clean launch
    latch_early()
    _, _, w2, fb2, m2 = run_step(ctx, w, inp, bad, cache.clone(), reset=True)
    ref_word, _, first, ref_msg = oracle.validate_indices(bad, inp["valid_len"])
    assert w2 == ref_word and fb2 == first[0] * (w.width + 1) + first[1] and m2 == ref_msg
    latch_early()
    _, _, w3, fb3, m3 = run_step(ctx, w, inp, bad, cache.clone(), reset=False)
    assert w3 == (ref_word | e_word) and (fb3, m3) == (e_fb, e_msg)  # the earlier first failure stays
    ctx.destroy()


def sa_bits(name):
    import sparse_attention_kv_append_amd as sa
    return getattr(sa, "SA_ERR_" + name)


def test_step_capacity_failure_appends_nothing():
    import torch
    w = CASES["decode_split"]
    banner("step capacity failure")
    inp, idx, cache = setup(w)
    inp = dict(inp)
    inp["past_len"] = inp["past_len"].copy()
    inp["past_len"][2] = w.cap  # batch 2 has no room for its current row
    ctx = make_ctx(w)
    c1, c2 = cache.clone(), cache.clone()
    _, pa, wa, _, _ = run_separate(ctx, w, inp, idx, c1)
    _, pb, wb, _, _ = run_step(ctx, w, inp, idx, c2)
    want = sa_bits("APPEND_CAPACITY") | sa_bits("APPEND_ANY")
    assert wa & want == want and wb & want == want
    assert torch.equal(c1, c2) and torch.equal(c2[2], cache[2])  # nothing appended for batch 2
    keep = [b for b in range(w.batch) if b != 2]
    assert torch.equal(pa[keep], pb[keep])
    ctx.destroy()


def test_step_graph_replays_match_eager():
    import torch
    w = CASES["decode_split"]
    banner("step graph capture")
    inp, idx, cache = setup(w)
    ctx = make_ctx(w)
    B = w.batch
    c_eager = cache.clone()
    y_eager, p_eager, w_eager, _, _ = run_step(ctx, w, inp, idx, c_eager)
    assert w_eager == 0
    c_g = cache.clone()
    plen, cur, q, ix = tt(inp["past_len"]), tt(inp["cur_k"]), tt(inp["q"]), tt(idx)
    prl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    y = torch.zeros((B, w.hq, w.q_seq, w.dv), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.step(q, B, w.q_seq, c_g, w.cap, plen, cur, w.cur, prl, ix, 1, w.width, y, reset_error=True)
    for rep in range(3):
        y.zero_()
        c_g.copy_(cache)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), rep
        assert torch.equal(c_g, c_eager) and torch.equal(prl, p_eager)
        assert ctx.read_error()[0] == 0
    ctx.destroy()


@pytest.mark.parametrize("name", ["decode_split", "long_cur"])
def test_rejected_step_launches_nothing(name):
    """A step the host rejects (index heads neither 1 nor Hq, a NULL query, an
    index width above the context's maximum) returns its status before the
    reset or the append is launched: the cache bytes, present_len and an
    earlier latched error word are all unchanged. long_cur takes the
    three-call form of the step, decode_split the one-launch form."""
    import torch
    import sparse_attention_kv_append_amd as sa
    w = CASES[name]
    banner(f"rejected step {name}")
    inp, idx, cache = setup(w)
    ctx = make_ctx(w)
    early = idx.copy()
    r = early[-1, 0, -1]
    r[1], r[2] = r[2], r[1]
    ctx.reset_error_async()
    ctx.validate_indices(tt(early), w.batch, 1, w.q_seq, w.width, valid_len=tt(inp["valid_len"]))
    e_word, e_fb, e_msg = ctx.read_error()
    assert e_word == (sa_bits("ORDER") | 512)
    B = w.batch
    c = cache.clone()
    plen, cur, q, ix = tt(inp["past_len"]), tt(inp["cur_k"]), tt(inp["q"]), tt(idx)
    prl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    y = torch.zeros((B, w.hq, w.q_seq, w.dv), dtype=torch.bfloat16, device="cuda")
    bad_calls = [
        (sa.SA_E_SHAPE, dict(q=q, index_heads=2, width=w.width)),
        (sa.SA_E_ARG, dict(q=None, index_heads=1, width=w.width)),
        (sa.SA_E_STATE, dict(q=q, index_heads=1, width=w.width + 1)),
    ]
    for status, kw in bad_calls:
        with pytest.raises(sa.SparseAttnError) as ei:
            ctx.step(kw["q"], B, w.q_seq, c, w.cap, plen, cur, w.cur, prl, ix, kw["index_heads"], kw["width"], y,
                     reset_error=True)
        assert ei.value.status == status, (ei.value.status, kw)
    torch.cuda.synchronize()
    assert torch.equal(c, cache)
    assert (prl == -7).all()
    assert ctx.read_error() == (e_word, e_fb, e_msg)
    ctx.destroy()


def test_inplace_append_with_mismatched_capacity_is_rejected():
    """In place (present aliases past) with past_capacity != present_capacity
    would read the new layout at the wrong row stride: SA_E_ARG, nothing written."""
    import torch
    import sparse_attention_kv_append_amd as sa
    w = CASES["decode_split"]
    banner("in-place append capacity mismatch")
    inp, idx, cache = setup(w)
    ctx = make_ctx(w)
    c = cache.clone()
    prl = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(sa.SparseAttnError) as ei:
        ctx.kv_append(w.batch, c, None, w.cap - 8, tt(inp["past_len"]), tt(inp["cur_k"]), None, w.cur, c, None,
                      w.cap, present_len=prl)
    assert ei.value.status == sa.SA_E_ARG
    torch.cuda.synchronize()
    assert torch.equal(c, cache) and (prl == -7).all()
    # the same call with matching capacities appends
    ctx.kv_append(w.batch, c, None, w.cap, tt(inp["past_len"]), tt(inp["cur_k"]), None, w.cur, c, None, w.cap,
                  present_len=prl)
    torch.cuda.synchronize()
    assert torch.equal(prl, tt(inp["valid_len"]))
    ctx.destroy()


def test_quantize_append_of_no_rows_writes_present_len():
    """fp8 quantize-on-append with cur_len == 0 still writes present_len
    (= past_len) and checks the capacity, as the byte-copy append does."""
    import torch
    w = CASES["fp8_split"]
    banner("fp8 quantize append of zero rows")
    inp, idx, cache = setup(w)
    ctx = make_ctx(w)
    c = cache.clone()
    prl = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
    ctx.reset_error_async()
    ctx.kv_append(w.batch, c, None, w.cap, tt(inp["past_len"]), tt(inp["cur_k"]), None, 0, c, None, w.cap,
                  present_len=prl, cur_is_unquantized_bf16=True)
    assert ctx.read_error()[0] == 0
    assert torch.equal(prl, tt(inp["past_len"])) and torch.equal(c, cache)
    # a past length beyond the capacity is latched, as on the copy path
    pl = inp["past_len"].copy()
    pl[1] = w.cap + 1
    ctx.kv_append(w.batch, c, None, w.cap, tt(pl), tt(inp["cur_k"]), None, 0, c, None, w.cap,
                  present_len=prl, cur_is_unquantized_bf16=True)
    want = sa_bits("APPEND_CAPACITY") | sa_bits("APPEND_ANY")
    assert ctx.read_error()[0] & want == want
    ctx.destroy()
