"""sparse_attn_step_kv (reset + in-place append of the current K/V rows +
forward with fused validation in one call) over separate K and V caches,
against the same three calls made separately, and against the oracle.

On the grouped-query MFMA path the step is one forward launch (plus the
split-KV combine) in which every workgroup writes its (batch, kv head)'s new
rows itself before it gathers, checks its share of the index columns, and the
launch's last arrival records the error block; the index rows below always
select the newest rows, so workgroups read rows they have just written. Y,
the cache bytes, present_len and the error word must equal those of the
separate calls bit for bit (same kernel arithmetic), including the reset
semantics, a bad index row and a capacity failure."""
import numpy as np
import pytest

import oracle
import sa_workloads as W
from gpu_support import check_close, make_ctx, tt

pytestmark = pytest.mark.gpu

GQA = W.WORKLOADS["dense_gqa"]
CASES = {
    # decode: 16 splits per (batch, kv head)
    "decode_split": GQA.scaled(batch=2, hq=32, hkv=8, q_seq=1, cur=1, past=3000, width=1200, topk=1100,
                               pattern="uniform", softcap=0.0, capacity=3100),
    "decode_softcap": GQA.scaled(batch=3, hq=16, hkv=4, q_seq=1, cur=1, past=1500, width=800, topk=760,
                                 pattern="uniform", capacity=1600),
    # several current rows, causal rows, query blocks of 32 (group 4)
    "prefill_rows": GQA.scaled(batch=2, hq=8, hkv=2, q_seq=40, cur=40, past=200, width=240, topk=240,
                               capacity=300),
    "group1": GQA.scaled(batch=2, hq=4, hkv=4, q_seq=5, cur=5, past=400, width=300, topk=290,
                         pattern="uniform", softcap=0.0, capacity=420),
}


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
    caches = []
    for name in ("past_k", "past_v"):
        c = torch.randint(-30000, 30000, (w.batch, w.hkv, w.cap, w.dk), dtype=torch.int16, device="cuda",
                          generator=gen)
        c[:, :, :w.past] = tt(inp[name][:, :, :w.past]).view(torch.int16)
        caches.append(c)
    return inp, idx, caches[0], caches[1]


def out_y(w):
    import torch
    return torch.full((w.batch, w.hq, w.q_seq, w.dv), float("nan"), dtype=torch.bfloat16, device="cuda")


def run_separate(ctx, w, inp, idx, kc, vc, plen, reset=True, i64=False):
    import torch
    prl = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
    y = out_y(w)
    if reset:
        ctx.reset_error_async()
    ctx.kv_append(w.batch, kc, vc, w.cap, plen, tt(inp["cur_k"]), tt(inp["cur_v"]), w.cur, kc, vc, w.cap,
                  present_len=prl)
    ctx.forward(tt(inp["q"]), w.batch, w.q_seq, kc, vc, w.cap, prl, tt(idx.astype(np.int64) if i64 else idx), 1,
                w.width, y, fused_validate=True)
    word, fb, msg = ctx.read_error()
    return y, prl, word, fb, msg


def run_step(ctx, w, inp, idx, kc, vc, plen, reset=True, i64=False):
    import torch
    prl = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
    y = out_y(w)
    ctx.step_kv(tt(inp["q"]), w.batch, w.q_seq, kc, vc, w.cap, plen, tt(inp["cur_k"]), tt(inp["cur_v"]), w.cur,
                prl, tt(idx.astype(np.int64) if i64 else idx), 1, w.width, y, reset_error=reset)
    word, fb, msg = ctx.read_error()
    return y, prl, word, fb, msg


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("i64", [False, True])
def test_step_kv_matches_separate_calls_and_oracle(name, i64):
    import torch
    w = CASES[name]
    banner(f"step_kv {name} i64={i64}")
    inp, idx, kc, vc = setup(w)
    ctx = make_ctx(w, idx64=i64)
    path, splits = ctx.query_plan(w.batch, w.q_seq, 1, w.width)
    assert path == 4
    plen = tt(inp["past_len"])
    k1, v1, k2, v2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    ya, pa, wa, _, ma = run_separate(ctx, w, inp, idx, k1, v1, plen, i64=i64)
    yb, pb, wb, _, mb = run_step(ctx, w, inp, idx, k2, v2, plen, i64=i64)
    assert wa == 0 and wb == 0, (ma, mb)
    assert torch.equal(pa, pb) and torch.equal(pb, tt(inp["valid_len"]))
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))
    pk = oracle.kv_append(inp["past_k"].copy(), inp["past_len"], inp["cur_k"])
    pv = oracle.kv_append(inp["past_v"].copy(), inp["past_len"], inp["cur_v"])
    got_k = k2[:, :, :w.total].cpu().numpy().view(np.uint16)
    assert np.array_equal(got_k, pk[:, :, :w.total])
    assert np.array_equal(v2[:, :, :w.total].cpu().numpy().view(np.uint16), pv[:, :, :w.total])
    assert torch.equal(k2[:, :, w.total:], kc[:, :, w.total:])  # spare rows untouched
    ref = oracle.forward(inp["q"], pk, pv, idx, q_dtype=w.dtype, cache_fmt=w.dtype, kv_layout=w.layout,
                         hkv=w.hkv, dv=w.dv, scale=w.scale, softcap=w.softcap, threads=8)
    check_close(yb.float().cpu().numpy(), ref, w.dtype, name)
    ctx.destroy()


def bad_rows(idx):
    out = idx.copy()
    out[0, 0, 0, 3] = out[0, 0, 0, 2]  # a duplicate in row 0
    r = out[-1, 0, -1]
    r[7], r[8] = r[8], r[7]            # an order violation in the last row
    return out


@pytest.mark.parametrize("name", ["decode_split", "prefill_rows"])
def test_step_kv_reset_semantics_and_verdict(name):
    """Without reset the step adds its bits to an earlier launch's; with reset
    it replaces them; a bad row's verdict (word, first failing position,
    message) equals the oracle validator's and the separate calls'."""
    w = CASES[name]
    banner(f"step_kv reset semantics {name}")
    inp, idx, kc, vc = setup(w)
    ctx = make_ctx(w)
    plen = tt(inp["past_len"])
    bad = bad_rows(idx)
    early = idx.copy()
    r = early[-1, 0, -1]
    r[1], r[2] = r[2], r[1]
    vl = tt(inp["valid_len"])

    def latch_early():
        ctx.reset_error_async()
        ctx.validate_indices(tt(early), w.batch, 1, w.q_seq, w.width, valid_len=vl)
        return ctx.read_error()

    e_word, e_fb, e_msg = latch_early()
    assert e_word != 0
    _, _, w0, fb0, m0 = run_step(ctx, w, inp, idx, kc.clone(), vc.clone(), plen, reset=False)
    assert (w0, fb0, m0) == (e_word, e_fb, e_msg)          # kept
    latch_early()
    _, _, w1, fb1, _ = run_step(ctx, w, inp, idx, kc.clone(), vc.clone(), plen, reset=True)
    assert w1 == 0 and fb1 == 2 ** 64 - 1                  # replaced by a clean launch
    ref_word, _, first, ref_msg = oracle.validate_indices(bad, inp["valid_len"])
    latch_early()
    _, _, w2, fb2, m2 = run_step(ctx, w, inp, bad, kc.clone(), vc.clone(), plen, reset=True)
    assert w2 == ref_word and fb2 == first[0] * (w.width + 1) + first[1] and m2 == ref_msg
    _, _, ws, fbs, ms = run_separate(ctx, w, inp, bad, kc.clone(), vc.clone(), plen, reset=True)
    assert (ws, fbs, ms) == (w2, fb2, m2)
    latch_early()
    _, _, w3, fb3, m3 = run_step(ctx, w, inp, bad, kc.clone(), vc.clone(), plen, reset=False)
    assert w3 == (ref_word | e_word) and (fb3, m3) == (e_fb, e_msg)  # the earlier first failure stays
    ctx.destroy()


def test_step_kv_capacity_failure_appends_nothing():
    """A batch entry whose past length leaves no room for the current rows:
    nothing is appended for it, present_len is not written for it, and the
    word carries the append bits, as in the separate calls."""
    import torch

    import sparse_attention_kv_append_amd as sa
    w = CASES["decode_split"]
    banner("step_kv capacity failure")
    inp, idx, kc, vc = setup(w)
    ctx = make_ctx(w)
    past = inp["past_len"].copy()
    past[1] = w.cap  # no room in batch entry 1
    plen = tt(past)
    k1, v1, k2, v2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    _, pa, wa, _, _ = run_separate(ctx, w, inp, idx, k1, v1, plen)
    _, pb, wb, _, _ = run_step(ctx, w, inp, idx, k2, v2, plen)
    want = sa.SA_ERR_APPEND_CAPACITY | sa.SA_ERR_APPEND_ANY
    assert wa & want == want and wb & want == want
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(k2[1], kc[1]) and torch.equal(v2[1], vc[1])
    assert int(pb[0].item()) == w.total and int(pa[0].item()) == w.total
    ctx.destroy()


def test_step_kv_graph_replays_match_eager():
    """The one-launch step captured in a HIP graph: every replay, with eager
    work between them, equals the eager call (Y, caches, present_len, word)."""
    import torch
    w = CASES["decode_split"]
    banner("step_kv graph replays")
    inp, idx, kc, vc = setup(w)
    ctx = make_ctx(w)
    plen = tt(inp["past_len"])
    ke, ve = kc.clone(), vc.clone()
    ye, pe, we, _, me = run_step(ctx, w, inp, idx, ke, ve, plen)
    assert we == 0, me
    k2, v2 = kc.clone(), vc.clone()
    q, ck, cv, ix = tt(inp["q"]), tt(inp["cur_k"]), tt(inp["cur_v"]), tt(idx)
    prl = torch.zeros((w.batch,), dtype=torch.int32, device="cuda")
    y = out_y(w)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.step_kv(q, w.batch, w.q_seq, k2, v2, w.cap, plen, ck, cv, w.cur, prl, ix, 1, w.width, y,
                    reset_error=True)
    for rep in range(3):
        y.zero_()
        prl.zero_()
        k2.copy_(kc)  # eager work between replays
        v2.copy_(vc)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ye.view(torch.int16)), rep
        assert torch.equal(prl, pe) and torch.equal(k2, ke) and torch.equal(v2, ve), rep
        word, _, msg = ctx.read_error()
        assert word == 0, msg
    ctx.destroy()


VERDICT_CASES = {
    # name: (workload, planting seed, planted column range)
    "split_decode": (GQA.scaled(batch=6, hq=32, hkv=8, q_seq=1, past=5000, cur=1, width=4000, topk=3900,
                                pattern="uniform", softcap=0.0, capacity=5100), 30, None),
    "split_decode_late": (GQA.scaled(batch=6, hq=32, hkv=8, q_seq=1, past=5000, cur=1, width=4000, topk=3990,
                                     pattern="uniform", softcap=0.0, capacity=5100), 31, (3700, 4000)),
    # 12 queries x group 4 = 48 rows per workgroup, causal rows of several current rows
    "rows_group4": (GQA.scaled(batch=2, hq=8, hkv=2, q_seq=12, past=500, cur=12, width=520, topk=520,
                               capacity=600), 32, None),
    # one kv head per query head: 32 queries per workgroup, three query blocks
    "group1_blocks": (GQA.scaled(batch=2, hq=4, hkv=4, q_seq=70, past=300, cur=70, width=380, topk=380,
                                 capacity=400), 33, None),
}


@pytest.mark.parametrize("name", list(VERDICT_CASES))
@pytest.mark.parametrize("i64", [False, True])
def test_step_kv_in_launch_verdict_matches_oracle(name, i64):
    """The one-launch step over index rows holding planted violations: the
    word, the first failing (row, column) and the message equal the oracle
    validator's against the appended lengths, on two launches in a row (the
    per-row slots re-arm)."""
    import torch

    from test_gpu_fused_verdicts import plant_violations
    w, seed, cols = VERDICT_CASES[name]
    banner(f"step_kv in-launch verdict {name} i64={i64}")
    inp, idx, kc, vc = setup(w)
    ctx = make_ctx(w, idx64=i64)
    assert ctx.query_plan(w.batch, w.q_seq, 1, w.width)[0] == 4
    bound = np.full(w.batch, w.total, np.int32)
    bad = plant_violations(W.index_rows(w, np.random.default_rng(seed)), bound, seed + 100 * i64, cols)
    if not i64:
        bad = bad.astype(np.int32)
    word, _, first, msg = oracle.validate_indices(bad, bound)
    assert word != 0
    plen = tt(inp["past_len"])
    for rep in range(2):
        _, prl, dword, dfirst, dmsg = run_step(ctx, w, inp, bad, kc.clone(), vc.clone(), plen, i64=i64)
        assert dword == word, f"launch {rep}: word {dword:#x} != {word:#x}"
        assert dfirst == first[0] * (w.width + 1) + first[1], f"launch {rep}"
        assert dmsg == msg
        assert torch.equal(prl, tt(inp["valid_len"]))
    ctx.destroy()
