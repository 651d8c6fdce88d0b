"""GPU parity of the grouped-query kernel (bf16 separate K/V caches of 128
dims, one index list per (batch, query)) against the oracle.

The kernel shares a gathered key tile among the queries of a workgroup when
their index rows agree column by column (or hold padding there) and redoes
any other tile one query at a time; the cases below cover both, their mix
inside one workgroup, several group sizes (1, 3, 4, 8, 32), ragged query
blocks, rows ending inside a tile, per-batch cache lengths, 64-bit indices and the softcap on and off."""
import numpy as np
import pytest

import oracle
import sa_workloads as W
from gpu_support import check_close, check_present, make_ctx, run_device, run_oracle

pytestmark = pytest.mark.gpu

GQA = W.WORKLOADS["dense_gqa"]


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


CASES = {
    # every query selects a causal prefix: all tiles shared
    "causal_group4": GQA.scaled(batch=2, hq=8, hkv=2, q_seq=40, past=600, cur=40, width=660, topk=660),
    # independent random selections: no tile shared
    "random_group4": GQA.scaled(batch=2, hq=8, hkv=2, q_seq=9, past=500, cur=9, width=310, topk=300,
                                pattern="uniform"),
    "causal_group1": GQA.scaled(batch=1, hq=3, hkv=3, q_seq=70, past=300, cur=70, width=380, topk=380),
    "causal_group3": GQA.scaled(batch=2, hq=6, hkv=2, q_seq=50, past=200, cur=50, width=260, topk=260,
                                softcap=0.0),
    "causal_group8": GQA.scaled(batch=1, hq=16, hkv=2, q_seq=37, past=100, cur=37, width=150, topk=150),
    "causal_group32": GQA.scaled(batch=1, hq=32, hkv=1, q_seq=7, past=90, cur=7, width=100, topk=100),
    "decode_group4": GQA.scaled(batch=3, hq=8, hkv=2, q_seq=1, past=333, cur=1, width=340, topk=200,
                                pattern="uniform"),
    # small softcaps, where c tanh(s / c) is far from s: softcap 1 saturates
    # most scores, softcap 12 bends a few
    "causal_softcap1": GQA.scaled(batch=2, hq=8, hkv=2, q_seq=40, past=600, cur=40, width=660, topk=660,
                                  softcap=1.0),
    "causal_softcap12": GQA.scaled(batch=2, hq=8, hkv=2, q_seq=40, past=600, cur=40, width=660, topk=660,
                                   softcap=12.0),
    "decode_softcap12": GQA.scaled(batch=3, hq=8, hkv=2, q_seq=1, past=333, cur=1, width=340, topk=200,
                                   pattern="uniform", softcap=12.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gqa_parity(name):
    w = CASES[name]
    banner(f"gqa parity {name}")
    ctx = make_ctx(w)
    assert ctx.query_plan(w.batch, w.q_seq, 1, w.width)[0] == 4
    ctx.destroy()
    inp = W.make_numpy(w)
    dev = run_device(w, inp)
    assert dev["word"] == 0, dev["msg"]
    y_ref, pk, pv = run_oracle(w, inp)
    check_present(w, dev, pk, pv)
    err = check_close(dev["y"], y_ref, w.dtype, name)
    banner(f"{name}: max |Y - oracle| = {err:.3e}")


def mixed_rows(w, rng):
    """Causal prefixes, except that some queries of each workgroup select
    random subsets and some end early."""
    idx = W.index_rows(w, rng)  # causal_all prefixes
    B, _, Sq, Wd = idx.shape
    T = w.total
    for b in range(B):
        for qi in range(Sq):
            k = qi % 7
            if k == 1:    # a random subset of its causal range
                pos = T - Sq + qi
                sel = np.sort(rng.choice(pos + 1, size=min(pos + 1, 57), replace=False))
                idx[b, 0, qi] = -1
                idx[b, 0, qi, :len(sel)] = sel
            elif k == 2:  # ends early, inside a tile
                n = int(rng.integers(1, 80))
                idx[b, 0, qi, n:] = -1
    return idx


@pytest.mark.parametrize("i64", [False, True])
def test_gqa_mixed_rows_and_ragged_lengths(i64):
    w = GQA.scaled(batch=2, hq=8, hkv=2, q_seq=45, past=400, cur=45, width=450, topk=450)
    banner(f"gqa mixed rows i64={i64}")
    inp = W.make_numpy(w)
    idx = mixed_rows(w, np.random.default_rng(5))
    # batch 1 appends after a shorter past: its valid length is 30 rows less
    # and its rows only select below it
    inp["past_len"] = np.array([w.past, w.past - 30], np.int32)
    vl = inp["past_len"] + w.cur
    inp["valid_len"] = vl
    idx[1][idx[1] >= vl[1]] = -1
    for qi in range(w.q_seq):  # keep the padding trailing after the cut
        row = idx[1, 0, qi]
        keep = row[row >= 0]
        row[:] = -1
        row[:len(keep)] = keep
    word, _, _, msg = oracle.validate_indices(idx, vl)
    assert word == 0, msg
    dev = run_device(w, inp, indices=idx, idx64=i64)
    assert dev["word"] == 0, dev["msg"]
    y_ref, pk, pv = run_oracle(w, inp, indices=idx)
    assert np.array_equal(dev["valid_len"], vl)
    err = check_close(dev["y"], y_ref, w.dtype, "gqa mixed")
    banner(f"gqa mixed: max |Y - oracle| = {err:.3e}")


SPLIT_CASES = {
    # few (batch, kv head) units: the key columns are split over several
    # workgroups and a combine merges their partial (max, sum, O)
    "decode_b1_long": GQA.scaled(batch=1, hq=8, hkv=2, q_seq=1, past=5000, cur=1, width=4000, topk=3900,
                                 pattern="uniform", softcap=0.0),
    # uneven last split, rows of different lengths (some end before the last splits)
    "decode_ragged": GQA.scaled(batch=2, hq=32, hkv=4, q_seq=1, past=3000, cur=1, width=1900, topk=1850,
                                pattern="uniform"),
    # several queries per workgroup, causal (shared tiles), with a split
    "causal_split": GQA.scaled(batch=1, hq=8, hkv=2, q_seq=12, past=1200, cur=12, width=1212, topk=1212),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_gqa_split_kv(name):
    """Split-KV decode: the plan splits, and Y equals the oracle's."""
    w = SPLIT_CASES[name]
    ctx = make_ctx(w)
    path, splits = ctx.query_plan(w.batch, w.q_seq, 1, w.width)
    banner(f"gqa split-kv {name}: path {path} splits {splits}")
    assert path == 4 and splits > 1
    inp = W.make_numpy(w)
    if name == "decode_ragged":
        # cut rows short: entries past a per-row length become -1 padding
        rng = np.random.default_rng(3)
        idx = inp["indices"]
        for b in range(w.batch):
            n = int(rng.integers(1, w.width))
            idx[b, 0, 0, n:] = -1
    dev = run_device(w, inp, ctx=ctx)
    ctx.destroy()
    assert dev["word"] == 0, dev["msg"]
    y_ref, pk, pv = run_oracle(w, inp)
    check_present(w, dev, pk, pv)
    err = check_close(dev["y"], y_ref, w.dtype, name)
    banner(f"{name}: max |Y - oracle| = {err:.3e}")
