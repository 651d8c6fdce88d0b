"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Present caches and validation verdicts must match bit for bit; Y must be
within |y - y_oracle| <= atol + rtol*|y_oracle| with (1e-5, 0) on the fp32
path and (2e-2, 1e-2) on the bf16 / fp8 paths.

Sizes here are the five workloads' structures shrunk so the oracle finishes
in seconds while still spanning several 32-key tiles, split-K with an empty
split, and ragged tails. Full-size launches are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest

import oracle
import sa_workloads as W
from gpu_support import (TOL, check_close, check_present, make_ctx, raw_bytes, run_device,
                         run_oracle, tt)

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


def scaled(name, **kw):
    return W.WORKLOADS[name].scaled(**kw)


CASES = {
    "tiny_f32": scaled("tiny_f32"),
    "tiny_f32_capacity": scaled("tiny_f32", capacity=80),
    "decode_bf16_small": scaled("decode_bf16", batch=3, past=1500, topk=700, width=710),
    "decode_bf16_two_tiles": scaled("decode_bf16", batch=5, past=90, topk=33, width=40),
    "decode_fp8_small": scaled("decode_fp8", batch=3, past=1200, topk=650, width=650),
    "prefill_small": scaled("prefill_bf16", q_seq=300, cur=300, width=128, topk=128),
    "dense_gqa_small": scaled("dense_gqa", batch=2, hq=8, hkv=2, q_seq=12, past=500, cur=12,
                              width=520, topk=520),
    "gqa_f16_per_head": scaled("dense_gqa", batch=2, hq=6, hkv=3, q_seq=3, past=200, cur=3,
                               width=150, topk=120, dtype=W.DT_F16, pattern="uniform",
                               index_heads=6, softcap=0.0),
    "mqa_generic_bf16": scaled("decode_bf16", batch=2, hq=16, past=300, topk=200, width=210),
    "fp8_generic_heads": scaled("decode_fp8", batch=2, hq=12, past=300, topk=100, width=128),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["inplace", "concat"])
def test_parity(name, mode):
    w = CASES[name]
    banner(f"parity {name} mode={mode}")
    inp = W.make_numpy(w)
    dev = run_device(w, inp, mode=mode)
    assert dev["word"] == 0, dev["msg"]
    y_ref, pk_ref, pv_ref = run_oracle(w, inp)
    check_present(w, dev, pk_ref, pv_ref)   # bit-exact, spare rows untouched
    assert np.array_equal(dev["valid_len"], inp["valid_len"])
    err = check_close(dev["y"], y_ref, w.dtype, name)
    banner(f"{name}: max |Y - oracle| = {err:.3e}")


def test_plan_selects_expected_paths():
    for name, want in [("decode_bf16_small", 2), ("prefill_small", 2), ("tiny_f32", 0),
                       ("dense_gqa_small", 4), ("mqa_generic_bf16", 0), ("decode_fp8_small", 3),
                       ("gqa_f16_per_head", 0)]:
        w = CASES[name]
        ctx = make_ctx(w)
        path, splits = ctx.query_plan(w.batch, w.q_seq, w.index_heads, w.width)
        assert path == want, name
        if name == "decode_bf16_small":
            assert splits > 1
        ctx.destroy()


def test_fp8_quantize_on_append_bit_exact():
    w = scaled("decode_fp8", batch=4, past=64, cur=5, q_seq=1, topk=40, width=48)
    banner("fp8 quantize-on-append")
    inp = W.make_numpy(w)
    # plant blocks that exercise zero, tiny, huge and tie cases in the current rows
    cur = (inp["cur_k"].astype(np.uint32) << 16).view(np.float32).copy()
    cur[0, 0, 0, 0:64] = 0.0
    cur[0, 0, 1, 64:128] *= np.float32(1e-30)
    cur[1, 0, 2, 128:192] *= np.float32(1e25)
    cur[2, 0, 3, 192:256] = np.float32(2.0) ** np.arange(-40, 24, dtype=np.float32)
    cur[3, 0, 4, 256:320] = -np.abs(cur[3, 0, 4, 256:320])
    import torch
    inp["cur_k"] = torch.from_numpy(cur).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for mode in ("inplace", "concat"):
        dev = run_device(w, inp, mode=mode, fp8_cur="bf16")
        assert dev["word"] == 0, dev["msg"]
        y_ref, rec_ref, _ = run_oracle(w, inp)
        check_present(w, dev, rec_ref, None)
        check_close(dev["y"], y_ref, w.dtype, "fp8 quantize-on-append")


def test_i64_indices_match_i32():
    w = CASES["decode_bf16_small"]
    inp = W.make_numpy(w)
    a = run_device(w, inp, idx64=False)
    b = run_device(w, inp, idx64=True)
    assert np.array_equal(a["y"], b["y"])
    w2 = CASES["dense_gqa_small"]
    inp2 = W.make_numpy(w2)
    assert np.array_equal(run_device(w2, inp2)["y"], run_device(w2, inp2, idx64=True)["y"])


@pytest.mark.parametrize("name", ["decode_bf16_small", "tiny_f32", "decode_fp8_small"])
def test_deterministic_reruns(name):
    w = CASES[name]
    inp = W.make_numpy(w)
    first = run_device(w, inp)
    for _ in range(3):
        again = run_device(w, inp)
        assert np.array_equal(raw_bytes(again["y"]), raw_bytes(first["y"]))
        assert np.array_equal(raw_bytes(again["present_k"]), raw_bytes(first["present_k"]))


@pytest.mark.parametrize("name", ["decode_bf16_small", "tiny_f32", "dense_gqa_small",
                                  "decode_fp8_small"])
def test_single_selected_key_returns_value_row_exactly(name):
    """With one selected key p = 1 exactly, so Y is that V row, bit for bit."""
    w = CASES[name]
    inp = W.make_numpy(w)
    idx = np.full_like(inp["indices"], -1)
    rng = np.random.default_rng(9)
    idx[..., 0] = rng.integers(0, w.total, size=idx.shape[:3])
    dev = run_device(w, inp, indices=idx)
    assert dev["word"] == 0, dev["msg"]
    y_ref, _, _ = run_oracle(w, inp, indices=idx)
    assert np.array_equal(dev["y"], y_ref)


@pytest.mark.parametrize("dtype", [W.DT_F16, W.DT_BF16])
def test_hi_one_equals_replicated_per_head_rows(dtype):
    """One index list per query equals the same list given to every head.
    In f16 both launches take the generic kernel: bit for bit. In bf16 one
    list per query takes the grouped-query kernel and per-head lists the
    generic one: both within the tolerance of the oracle."""
    w = CASES["dense_gqa_small"].scaled(dtype=dtype)
    inp = W.make_numpy(w)
    a = run_device(w, inp)
    rep = np.ascontiguousarray(np.repeat(inp["indices"], w.hq, axis=1))
    wr = w.scaled(index_heads=w.hq)
    b = run_device(wr, inp, indices=rep)
    if dtype == W.DT_F16:
        assert np.array_equal(a["y"], b["y"])
    else:
        y_ref, _, _ = run_oracle(w, inp)
        check_close(a["y"], y_ref, dtype, "one list per query")
        check_close(b["y"], y_ref, dtype, "one list per head")


def test_prefill_chain_present_feeds_next_decode():
    """Prefill then two decode steps, each present fed back as the next past."""
    base = scaled("decode_bf16", batch=2, past=0, cur=40, q_seq=1, topk=30, width=32,
                  capacity=48, pattern="uniform")
    ctx = make_ctx(base, max_q_seq=40)
    import torch
    rng = np.random.default_rng(21)
    cache = tt(np.zeros((2, 1, 48, 576), np.uint16))
    host = np.zeros((2, 1, 48, 576), np.uint16)
    plen = np.zeros(2, np.int32)
    for step, cur_len in enumerate([40, 1, 1]):
        w = base.scaled(past=int(plen[0]), cur=cur_len, seed=100 + step)
        inp = W.make_numpy(w)
        inp["past_k"] = host.copy()
        inp["past_len"] = plen.copy()
        vlen = torch.zeros(2, dtype=torch.int32, device="cuda")
        ctx.reset_error_async()
        ctx.kv_append(2, cache, None, 48, tt(plen), tt(inp["cur_k"]), None, cur_len, cache, None, 48,
                      present_len=vlen)
        total = int(plen[0]) + cur_len
        idx = np.full((2, 1, 1, 32), -1, np.int32)
        for b in range(2):
            k = min(30, total)
            idx[b, 0, 0, :k] = np.sort(rng.choice(total, size=k, replace=False))
        y = torch.empty((2, 64, 1, 512), dtype=torch.bfloat16, device="cuda")
        ctx.forward(tt(inp["q"]), 2, 1, cache, None, 48, vlen, tt(idx), 1, 32, y, fused_validate=True)
        word, _, msg = ctx.read_error()
        assert word == 0, msg
        host = oracle.kv_append(host.copy(), plen, inp["cur_k"])
        assert np.array_equal(raw_bytes(cache.cpu().numpy()), raw_bytes(host))
        ref = oracle.forward(inp["q"], host, None, idx, q_dtype=W.DT_BF16, cache_fmt=W.DT_BF16,
                             kv_layout=1, hkv=1, dv=512, scale=w.scale)
        check_close(y.float().cpu().numpy(), ref, W.DT_BF16, f"chain step {step}")
        plen = plen + cur_len
    ctx.destroy()


def test_append_capacity_errors():
    w = scaled("tiny_f32")
    ctx = make_ctx(w)
    import torch
    import sparse_attention_kv_append_amd as sa
    inp = W.make_numpy(w)
    kc, vc = tt(inp["past_k"]), tt(inp["past_v"])
    before = raw_bytes(kc.cpu().numpy()).copy()
    # host-visible: dense past (past_len NULL) + current exceeds capacity
    with pytest.raises(sa.SparseAttnError) as ei:
        ctx.kv_append(1, kc, vc, 64, None, tt(inp["cur_k"]), tt(inp["cur_v"]), 4, kc, vc, 64)
    assert ei.value.status == sa.SA_E_CAPACITY
    # device-visible: past_len 62 + 4 > 64 latches and writes nothing
    ctx.reset_error_async()
    ctx.kv_append(1, kc, vc, 64, tt(np.array([62], np.int32)), tt(inp["cur_k"]), tt(inp["cur_v"]),
                  4, kc, vc, 64)
    word, _, msg = ctx.read_error()
    assert word & sa.SA_ERR_APPEND_CAPACITY and "capacity" in msg
    assert np.array_equal(raw_bytes(kc.cpu().numpy()), before)
    ctx.destroy()


def test_graph_capture_replays_match_eager():
    """reset + append + validate + forward captured in a HIP graph; every replay
    (with eager work and synchronisations between replays) equals the eager
    result, and the error word read after each replay is clean."""
    import torch
    w = CASES["decode_bf16_small"]
    inp = W.make_numpy(w)
    ctx = make_ctx(w)
    cache = tt(inp["past_k"])
    cur = tt(inp["cur_k"])
    plen = tt(inp["past_len"])
    vlen = torch.zeros_like(plen)
    q = tt(inp["q"])
    idx = tt(inp["indices"])
    y = torch.empty((w.batch, w.hq, 1, w.dv), dtype=torch.bfloat16, device="cuda")

    def step():
        ctx.reset_error_async()
        ctx.kv_append(w.batch, cache, None, w.cap, plen, cur, None, 1, cache, None, w.cap,
                      present_len=vlen)
        ctx.forward(q, w.batch, 1, cache, None, w.cap, vlen, idx, 1, w.width, y, fused_validate=True)

    step()
    torch.cuda.synchronize()
    eager = y.clone()
    assert ctx.read_error()[0] == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        y.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        assert ctx.read_error()[0] == 0
        del junk
    # a poisoned index set seen by a replay latches the word; outputs stay finite
    bad = inp["indices"].copy()
    bad[0, 0, 0, 5] = bad[0, 0, 0, 4]
    idx.copy_(tt(bad))
    g.replay()
    word, _, msg = ctx.read_error()
    assert word & 0x08 and "duplicate" in msg
    assert torch.isfinite(y.float()).all()
    ctx.destroy()


def planted_records(w, inp, seed):
    """Oracle records of the generator's rows with planted bytes: blocks whose
    scale byte is outside the range the fast hardware decode covers (3..9 with
    their codes; 247..250 with only +0 / -0 codes, since any other code would
    overflow the scores), and blocks carrying every finite E4M3FN code
    (subnormals, zeros, both signs) at the block's own scale."""
    rng = np.random.default_rng(seed)
    past = oracle_records_of(inp["past_k"], w)
    cur = oracle_records_of(inp["cur_k"], w)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    for rec in (past[:, :, :w.past], cur):
        flat = rec.reshape(-1, rec.shape[-1])
        for r in range(flat.shape[0]):
            for j in range(8):
                kind = rng.integers(0, 4)
                blk = flat[r, 65 * j: 65 * j + 65]
                if kind == 0:      # every finite code, shuffled
                    blk[1:] = rng.permutation(finite)[:64]
                elif kind == 1:    # tiny scale: values near the bottom of fp32 normals
                    blk[0] = rng.integers(3, 10)
                elif kind == 2:    # huge scale, signed zeros only
                    blk[0] = rng.integers(247, 251)
                    blk[1:] = rng.integers(0, 2, size=64).astype(np.uint8) << 7
    return past, cur


def oracle_records_of(bits, w):
    from gpu_support import oracle_records
    return oracle_records(bits, w)


@pytest.mark.parametrize("single", [False, True])
def test_fp8_planted_scales_and_codes(single):
    """fp8 records with planted scale bytes and codes through the wave-pair
    kernel: every block decodes like the oracle's record decoder."""
    w = scaled("decode_fp8", batch=2, past=200, topk=96, width=100)
    banner(f"fp8 planted records single={single}")
    inp = W.make_numpy(w)
    recs = planted_records(w, inp, 5)
    idx = None
    if single:
        idx = np.full_like(inp["indices"], -1)
        idx[..., 0] = np.random.default_rng(6).integers(0, w.total, size=idx.shape[:3])
    dev = run_device(w, inp, records=recs, indices=idx)
    assert dev["word"] == 0, dev["msg"]
    y_ref, rec_ref, _ = run_oracle(w, inp, records=recs, indices=idx)
    check_present(w, dev, rec_ref, None)
    check_close(dev["y"], y_ref, w.dtype, "planted fp8 records")
    if single:
        # p = 1 exactly: Y is the decoded V row; bf16-normal values are exact
        big = np.abs(y_ref) >= 2.0 ** -126
        assert np.array_equal(dev["y"][big], y_ref[big])


@pytest.mark.parametrize("name", ["decode_bf16_small", "prefill_small"])
def test_huge_late_scores_restart_and_match(name):
    """A key whose score is about 2^100 above the first tile's maximum sits in a
    later tile: the shared-latent kernel redoes its key range with the larger
    reference and still matches the oracle (no overflow to inf / NaN)."""
    w = CASES[name]
    inp = W.make_numpy(w)
    k = inp["past_k"].copy()
    f32 = (k.astype(np.uint32) << 16).view(np.float32)
    idx = inp["indices"]
    b, qi = 0, w.q_seq - 1
    row = idx[b, 0, qi]
    key = int(row[row >= 0][-1])  # the row's last selected key: a late tile
    if key < w.past:
        f32[b, 0, key, :64] = np.float32(3.0e4)
        inp["past_k"] = (f32.view(np.uint32) >> 16).astype(np.uint16)
    else:
        c = (inp["cur_k"].astype(np.uint32) << 16).view(np.float32).copy()
        c[b, 0, key - w.past, :64] = np.float32(3.0e4)
        inp["cur_k"] = (c.view(np.uint32) >> 16).astype(np.uint16)
    dev = run_device(w, inp)
    assert dev["word"] == 0, dev["msg"]
    y_ref, _, _ = run_oracle(w, inp)
    assert np.isfinite(y_ref).all()
    check_close(dev["y"], y_ref, w.dtype, f"huge late score {name}")

