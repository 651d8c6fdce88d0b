"""GPU parity of the optional attention bias (sparse_attn_forward_bias) and
capacity-mode length recovery (sparse_attn_capacity_lengths), through the C
ABI, against the oracle on the same seeded inputs.

Bar: lengths and write positions bit-exact (integer); the in-place present
byte-identical to the oracle's append at the recovered write positions; Y
within the floating tolerance of its dtype (f32 1e-5; bf16/f16 2e-2 + 1e-2
relative); the error word zero on valid inputs.
"""
import numpy as np
import pytest

import oracle
import sa_workloads as W
from gpu_support import check_close, make_ctx, oracle_records, raw_bytes, to_np, tt, y_as_f32, y_dtype

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


def present_host(inp):
    pk = oracle.kv_append(inp["past_k"].copy(), inp["past_len"], inp["cur_k"])
    pv = None if inp["past_v"] is None else oracle.kv_append(inp["past_v"].copy(), inp["past_len"], inp["cur_v"])
    return pk, pv


def bias_store(b32, dtype):
    if dtype == W.DT_F32:
        return np.ascontiguousarray(b32, np.float32)
    if dtype == W.DT_F16:
        return np.ascontiguousarray(b32, np.float32).astype(np.float16).view(np.uint16)
    return oracle.bf16_bits(np.ascontiguousarray(b32, np.float32))


def run_bias(w, inp, bias, *, fp8=False, idx64=False, path=None):
    """Device forward_bias over the oracle's present; returns (y, word, msg).
    With `path`, the configuration's plan must name that kernel."""
    import torch
    pk, pv = present_host(inp)
    kc = oracle_records(pk, w) if fp8 else pk
    ctx = make_ctx(w, idx64=idx64)
    if path is not None:
        assert ctx.query_plan(w.batch, w.q_seq, inp["indices"].shape[1], w.width)[0] == path
    y = torch.full((w.batch, w.hq, w.q_seq, w.dv), float("nan"), dtype=y_dtype(w), device="cuda")
    vl = torch.tensor(np.full(w.batch, w.total, np.int32), device="cuda")
    idx = inp["indices"].astype(np.int64) if idx64 else inp["indices"]
    ctx.reset_error_async()
    ctx.forward_bias(tt(inp["q"]), w.batch, w.q_seq, tt(kc), None if pv is None else tt(pv), w.cap, vl,
                     tt(idx), inp["indices"].shape[1], w.width, None if bias is None else tt(bias),
                     y, fused_validate=True)
    word, _, msg = ctx.read_error()
    ctx.destroy()
    return y_as_f32(y), word, msg


def oracle_bias(w, inp, bias, *, fp8=False):
    pk, pv = present_host(inp)
    kc, fmt = (oracle_records(pk, w), oracle.FP8_BLOCK64) if fp8 else (pk, w.dtype)
    return oracle.forward(inp["q"], kc, pv, inp["indices"], q_dtype=w.dtype, cache_fmt=fmt,
                          kv_layout=w.layout, hkv=w.hkv, dv=w.dv, rope=w.rope, scale=w.scale,
                          softcap=w.softcap, bias=bias, threads=8)


CASES = {
    "tiny_f32": W.WORKLOADS["tiny_f32"].scaled(batch=2),
    "grouped_bf16_per_head": W.WORKLOADS["dense_gqa"].scaled(batch=2, hq=8, hkv=2, q_seq=3, past=200, cur=3,
                                                             width=120, topk=100, pattern="uniform",
                                                             index_heads=8, softcap=0.0),
    "gqa_softcap_f16": W.WORKLOADS["dense_gqa"].scaled(batch=2, hq=8, hkv=2, q_seq=5, past=300, cur=5,
                                                       width=305, topk=305, dtype=W.DT_F16),
    # bf16, 128 dims, one index list per query: the grouped-query MFMA kernel
    "gqa_causal_softcap": W.WORKLOADS["dense_gqa"].scaled(batch=2, hq=8, hkv=2, q_seq=12, past=500, cur=12,
                                                          width=512, topk=512),
    "gqa_uniform_decode": W.WORKLOADS["dense_gqa"].scaled(batch=3, hq=16, hkv=4, q_seq=1, past=3000, cur=1,
                                                          width=700, topk=650, pattern="uniform", softcap=0.0),
    "gqa_uniform_rows": W.WORKLOADS["dense_gqa"].scaled(batch=2, hq=4, hkv=2, q_seq=3, past=400, cur=3,
                                                        width=100, topk=90, pattern="uniform", softcap=0.0),
    "fp8_records": W.WORKLOADS["decode_fp8"].scaled(batch=2, hq=16, past=300, topk=100, width=128),
    "latent_bf16": W.WORKLOADS["decode_bf16"].scaled(batch=3, hq=16, past=400, topk=260, width=300),
    # 64 heads of 576 / 512 dims: the shared-latent MFMA kernels (plan path 2
    # bf16 rows, 3 fp8 records), split over several workgroups per row and
    # merged by the combine, or one workgroup per row
    "latent_mfma_split": W.WORKLOADS["decode_bf16"].scaled(batch=3, past=1500, topk=700, width=710,
                                                           capacity=1600),
    "latent_mfma_rows": W.WORKLOADS["decode_bf16"].scaled(batch=1, q_seq=40, cur=40, past=600, topk=500,
                                                          width=520, capacity=700),
    "latent_mfma_softcap": W.WORKLOADS["decode_bf16"].scaled(batch=2, past=900, topk=400, width=400,
                                                             capacity=1000, softcap=30.0),
    "fp8_pair_split": W.WORKLOADS["decode_fp8"].scaled(batch=2, past=1200, topk=650, width=650, capacity=1300),
    "fp8_pair_rows": W.WORKLOADS["decode_fp8"].scaled(batch=1, q_seq=40, cur=40, past=400, topk=300,
                                                      width=300, capacity=500),
}
MFMA_PATH = {"latent_mfma_split": 2, "latent_mfma_rows": 2, "latent_mfma_softcap": 2, "fp8_pair_split": 3,
             "fp8_pair_rows": 3}
SHAPES = ["full", "b11k", "sk", "h11", "scalar"]


def make_bias(w, shape, seed=3, holes=True):
    dims = {"full": (w.batch, w.hq, w.q_seq, w.cap), "b11k": (w.batch, 1, 1, w.cap), "sk": (w.q_seq, w.cap),
            "h11": (w.hq, 1, 1), "scalar": ()}[shape]
    rng = np.random.default_rng(seed)
    b = rng.standard_normal(dims).astype(np.float32)
    if holes and b.ndim and b.shape[-1] == w.cap:
        b[rng.random(dims) < 0.15] = -np.inf
    return bias_store(b, w.dtype)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("shape", SHAPES)
def test_forward_bias_matches_oracle(name, shape):
    w = CASES[name]
    fp8 = w.cache_format == W.CACHE_FP8
    inp = W.make_numpy(w)
    bias = make_bias(w, shape)
    banner(f"forward_bias {name} bias {shape} {bias.shape}")
    ref = oracle_bias(w, inp, bias, fp8=fp8)
    y, word, msg = run_bias(w, inp, bias, fp8=fp8, path=MFMA_PATH.get(name))
    assert word == 0, msg
    check_close(y, ref, w.dtype, f"{name}/{shape}")


@pytest.mark.parametrize("name", ["latent_mfma_split", "fp8_pair_rows"])
def test_forward_bias_mfma_int64_indices(name):
    w = CASES[name]
    fp8 = w.cache_format == W.CACHE_FP8
    inp = W.make_numpy(w)
    bias = make_bias(w, "full", seed=4)
    banner(f"forward_bias {name} int64 indices")
    ref = oracle_bias(w, inp, bias, fp8=fp8)
    y, word, msg = run_bias(w, inp, bias, fp8=fp8, idx64=True, path=MFMA_PATH[name])
    assert word == 0, msg
    check_close(y, ref, w.dtype, f"{name}/i64")


@pytest.mark.parametrize("name", ["latent_mfma_split", "fp8_pair_split"])
def test_forward_bias_mfma_flags_bad_index(name):
    """A biased call on the shared-latent kernels still validates its index
    rows in the launch: the word and the first failing column equal the
    oracle's."""
    w = CASES[name]
    fp8 = w.cache_format == W.CACHE_FP8
    inp = W.make_numpy(w)
    inp["indices"][1, 0, 0, 5] = inp["indices"][1, 0, 0, 4]  # a repeated key: not strictly increasing
    word_ref, _, _, _ = oracle.validate_indices(inp["indices"], np.full(w.batch, w.total, np.int32))
    assert word_ref != 0
    y, word, msg = run_bias(w, inp, make_bias(w, "b11k"), fp8=fp8, path=MFMA_PATH[name])
    assert word == word_ref, msg


def test_forward_bias_none_is_the_plain_forward():
    w = CASES["tiny_f32"]
    inp = W.make_numpy(w)
    ref = oracle_bias(w, inp, None)
    y, word, msg = run_bias(w, inp, None)
    assert word == 0, msg
    check_close(y, ref, w.dtype, "no bias")


@pytest.mark.parametrize("name", ["grouped_bf16_per_head", "gqa_uniform_decode", "gqa_causal_softcap",
                                  "latent_mfma_split", "latent_mfma_rows", "fp8_pair_split", "fp8_pair_rows"])
def test_forward_bias_masked_rows_give_zeros(name):
    """Rows whose every key is masked give zeros (generic kernel; grouped-query
    kernel with and without split-KV; the shared-latent kernels with and
    without splits)."""
    w = CASES[name]
    fp8 = w.cache_format == W.CACHE_FP8
    inp = W.make_numpy(w)
    b32 = np.zeros((w.batch, w.hq, w.q_seq, 1), np.float32)
    last = (min(1, w.batch - 1), 3, w.q_seq - 1)
    b32[last] = -np.inf
    b32[0, :, 0] = -np.inf
    bias = bias_store(b32, w.dtype)
    ref = oracle_bias(w, inp, bias, fp8=fp8)
    assert not ref[last].any() and not ref[0, :, 0].any()
    y, word, msg = run_bias(w, inp, bias, fp8=fp8, path=MFMA_PATH.get(name))
    assert word == 0, msg
    assert not y[last].any() and not y[0, :, 0].any()
    check_close(y, ref, w.dtype, "masked rows")


def test_bias_host_errors():
    import torch

    import sparse_attention_kv_append_amd as sa
    w = CASES["tiny_f32"]
    ctx = make_ctx(w)
    dev = "cuda"
    q = torch.zeros((w.batch, w.hq, w.q_seq, w.dk), device=dev)
    k = torch.zeros((w.batch, w.hkv, w.cap, w.dk), device=dev)
    idx = torch.zeros((w.batch, 1, w.q_seq, w.width), dtype=torch.int32, device=dev)
    y = torch.zeros_like(q)
    vl = torch.zeros(w.batch, dtype=torch.int32, device=dev)
    for bad in [(1, 1, 1, 1, 1), (3, 1, 1, 1), (w.cap + 1,), (1, 2, 1, 1)]:
        with pytest.raises(sa.SparseAttnError) as e:
            ctx.forward_bias(q, w.batch, w.q_seq, k, k, w.cap, vl, idx, 1, w.width,
                             torch.zeros(bad, device=dev), y)
        assert e.value.status == sa.SA_E_SHAPE, bad
    with pytest.raises(sa.SparseAttnError) as e:
        ctx.capacity_lengths(torch.zeros((w.cap + 2,), device=dev), w.batch, w.q_seq, w.cap, 1, vl, vl)
    assert e.value.status == sa.SA_E_SHAPE
    assert ctx.lib.sparse_attn_capacity_lengths(ctx.handle, None, None, 0, w.batch, w.q_seq, w.cap, 1,
                                                vl.data_ptr(), vl.data_ptr()) == sa.SA_E_ARG
    cur = torch.zeros((w.batch, w.hkv, 1, w.dk), device=dev)
    for bad_bias, cur_len, status in [(torch.zeros((1, 1, 1, 1, 1), device=dev), 1, sa.SA_E_SHAPE),
                                      (torch.zeros((w.cap,), device=dev), 0, sa.SA_E_CAPACITY),
                                      (torch.zeros((w.cap,), device=dev), w.cap + 1, sa.SA_E_CAPACITY)]:
        with pytest.raises(sa.SparseAttnError) as e:
            ctx.capacity_step(q, w.batch, w.q_seq, k, k.clone(), w.cap, cur, cur, cur_len, idx, 1, w.width,
                              bad_bias, y, vl, vl)
        assert e.value.status == status
    ctx.destroy()
    # separate caches need both V tensors
    ctx = make_ctx(w)
    with pytest.raises(sa.SparseAttnError) as e:
        ctx.capacity_step(q, w.batch, w.q_seq, k, None, w.cap, cur, cur, 1, idx, 1, w.width,
                          torch.zeros((w.cap,), device=dev), y, vl, vl)
    assert e.value.status == sa.SA_E_ARG
    ctx.destroy()
    wl = W.WORKLOADS["decode_bf16"].scaled(batch=1, past=10, width=8, topk=8)
    ctx = make_ctx(wl)  # a shared-latent cache takes no V tensors
    with pytest.raises(sa.SparseAttnError) as e:
        ctx.capacity_step(q, 1, 1, k, k, w.cap, cur, cur, 1, idx, 1, 8, torch.zeros((w.cap,), device=dev), y, vl, vl)
    assert e.value.status == sa.SA_E_ARG
    ctx.destroy()


@pytest.mark.parametrize("dtype,shape", [(W.DT_F32, (3, 8, 2, 300)), (W.DT_F32, (3, 1, 1, 300)),
                                         (W.DT_BF16, (300,)), (W.DT_BF16, (3, 1, 2, 300)),
                                         (W.DT_F16, (1, 8, 1, 300)), (W.DT_F32, (3, 8, 2, 1)),
                                         # rows of whole 16-byte vectors: the vector path
                                         (W.DT_BF16, (3, 1, 2, 320)), (W.DT_F16, (1, 8, 2, 4096)),
                                         (W.DT_F32, (3, 8, 1, 4100)), (W.DT_BF16, (16384,)),
                                         # long rows that are not whole vectors: scanned from the
                                         # end in batches of 4096 vectors, loose elements at both ends
                                         (W.DT_BF16, (70001,)), (W.DT_F32, (3, 1, 1, 40001)),
                                         (W.DT_F16, (1, 8, 2, 32769))])
def test_capacity_lengths_match_oracle(dtype, shape):
    import torch
    cap = shape[-1] if shape[-1] > 1 else 300
    w = W.CAPACITY_WORKLOADS["capacity_small"].scaled(dtype=dtype, capacity=cap)
    rng = np.random.default_rng(12)
    b32 = rng.standard_normal(shape).astype(np.float32)
    lead = b32.reshape(-1, shape[-1])
    for i in range(lead.shape[0]):
        f = int(rng.integers(0, shape[-1] + 1))
        lead[i, f:] = -np.inf
        lead[i, rng.integers(0, shape[-1], 3)] = np.nan
    if len(shape) == 4 and shape[0] == 3:
        b32[1] = -np.inf      # no live row in batch entry 1
    bias = bias_store(b32, dtype)
    banner(f"capacity_lengths dtype {dtype} shape {shape}")
    for cur in (1, 2, 250):
        valid, wpos = oracle.capacity_lengths(bias, w.cap, cur, batch=w.batch, heads=w.hq, q_seq=w.q_seq,
                                              bias_dtype=dtype)
        ctx = make_ctx(w)
        vl = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
        wp = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
        ctx.capacity_lengths(tt(bias), w.batch, w.q_seq, w.cap, cur, vl, wp)
        np.testing.assert_array_equal(to_np(vl), valid)
        np.testing.assert_array_equal(to_np(wp), wpos)
        ctx.destroy()


def capacity_oracle(w, inp):
    valid, wpos = oracle.capacity_lengths(inp["bias"], w.cap, w.cur, batch=w.batch, heads=w.hq, q_seq=w.q_seq,
                                          bias_dtype=w.dtype)
    assert np.array_equal(valid, inp["valid"])
    word, _, _, _ = oracle.validate_indices(inp["indices"], valid)
    assert word == 0
    pk = oracle.kv_append(inp["past_k"].copy(), wpos, inp["cur_k"])
    pv = oracle.kv_append(inp["past_v"].copy(), wpos, inp["cur_v"])
    return valid, wpos, pk, pv


def capacity_device(w, inp, ctx=None, one_call=False):
    """capacity_lengths -> in-place kv_append at write_pos -> forward_bias with
    fused validation against valid_len, all on the context's stream."""
    import torch
    own = ctx is None
    if own:
        ctx = make_ctx(w)
    kc, vc = tt(inp["past_k"]), tt(inp["past_v"])
    bias = tt(inp["bias"])
    vl = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
    wp = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
    y = torch.full((w.batch, w.hq, w.q_seq, w.dv), float("nan"), dtype=y_dtype(w), device="cuda")
    if one_call:
        ctx.capacity_step(tt(inp["q"]), w.batch, w.q_seq, kc, vc, w.cap, tt(inp["cur_k"]), tt(inp["cur_v"]), w.cur,
                          tt(inp["indices"]), 1, w.width, bias, y, vl, wp, reset_error=True)
    else:
        ctx.reset_error_async()
        ctx.capacity_lengths(bias, w.batch, w.q_seq, w.cap, w.cur, vl, wp)
        ctx.kv_append(w.batch, kc, vc, w.cap, wp, tt(inp["cur_k"]), tt(inp["cur_v"]), w.cur, kc, vc, w.cap)
        ctx.forward_bias(tt(inp["q"]), w.batch, w.q_seq, kc, vc, w.cap, vl, tt(inp["indices"]), 1, w.width, bias, y,
                         fused_validate=True)
    word, _, msg = ctx.read_error()
    out = dict(valid=to_np(vl), wpos=to_np(wp), k=to_np(kc), v=to_np(vc), y=y_as_f32(y), word=word, msg=msg)
    if own:
        ctx.destroy()
    return out


@pytest.mark.parametrize("kw", [dict(), dict(dtype=W.DT_BF16, seed=8), dict(q_seq=1, cur=1, seed=9),
                                dict(batch=2, hq=4, hkv=4, q_seq=4, cur=4, width=300, topk=300, seed=10),
                                # bf16 with 128 dims: the grouped-query kernel
                                dict(dtype=W.DT_BF16, dk=128, dv=128, q_seq=1, cur=1, seed=11),
                                dict(dtype=W.DT_BF16, dk=128, dv=128, hq=16, hkv=2, seed=12),
                                # rows not a multiple of 16 bytes: the one-call step takes the two launches
                                dict(dk=66, dv=66, seed=13), dict(dtype=W.DT_BF16, dk=72, dv=72, seed=14)])
@pytest.mark.parametrize("one_call", [False, True])
def test_capacity_step_matches_oracle(kw, one_call):
    """The capacity step as four calls and as sparse_attn_capacity_step."""
    w = W.CAPACITY_WORKLOADS["capacity_small"].scaled(**kw)
    inp = W.make_capacity_numpy(w)
    banner(f"capacity step {w.name} {kw} one_call={one_call}")
    valid, wpos, pk, pv = capacity_oracle(w, inp)
    ref = oracle.forward(inp["q"], pk, pv, inp["indices"], q_dtype=w.dtype, cache_fmt=w.dtype,
                         kv_layout=w.layout, hkv=w.hkv, dv=w.dv, scale=w.scale, bias=inp["bias"], threads=8)
    d = capacity_device(w, inp, one_call=one_call)
    assert d["word"] == 0, d["msg"]
    np.testing.assert_array_equal(d["valid"], valid)
    np.testing.assert_array_equal(d["wpos"], wpos)
    assert np.array_equal(raw_bytes(d["k"]), raw_bytes(pk)) and np.array_equal(raw_bytes(d["v"]), raw_bytes(pv))
    check_close(d["y"], ref, w.dtype, "capacity step")


@pytest.mark.parametrize("name", ["capacity_decode", "capacity_latent_decode"])
def test_capacity_decode_fullsize_sampled_rows(name):
    """The benchmark's capacity-mode decodes (batch 32, 32 q heads / 8 kv heads,
    head dim 128, capacity 16384, top-2048, bf16; and the shared-latent one:
    64 heads over one 576-dim row, capacity 32769) in their launch
    configuration: lengths and write positions exact, the appended rows
    exact, Y of sampled batch entries (all heads) against the oracle's
    capacity step on those entries."""
    import torch

    import bench
    banner(f"{name} full size: building inputs")
    s = bench.CapacitySetup(name, 1)
    assert s.path == (2 if name == "capacity_latent_decode" else 4)
    s.step(0)
    torch.cuda.synchronize()
    word, _, msg = s.ctx.read_error()
    assert word == 0, msg
    w = s.w
    vl, wp = to_np(s.vl), to_np(s.wp)
    y = y_as_f32(s.y)
    for b in [0, 7, 19, 31]:
        banner(f"{name} full size: oracle on batch entry {b}")
        inp = s.oracle_inputs(b)
        ref, valid, wpos = s.oracle_y(inp, 8)
        assert vl[b] == valid[0] and wp[b] == wpos[0]
        kb = s.k[b:b + 1, :, wpos[0]:wpos[0] + w.cur].contiguous().view(torch.int16).cpu().numpy()
        np.testing.assert_array_equal(kb.view(np.uint16), inp["cur_k"])
        check_close(y[b:b + 1], ref, w.dtype, f"batch entry {b}")
    s.ctx.destroy()


def test_capacity_step_graph_replays_match_eager():
    """sparse_attn_capacity_step captured in a HIP graph (lengths + append
    launch, validation, grouped-query forward with bias and split-KV, combine):
    every replay, with eager work between them, equals the eager call."""
    import torch
    w = W.CAPACITY_WORKLOADS["capacity_small"].scaled(dtype=W.DT_BF16, dk=128, dv=128, q_seq=1, cur=1,
                                                      capacity=2000, width=600, topk=560, seed=21,
                                                      extra={"valid_lo": 900})
    inp = W.make_capacity_numpy(w)
    ctx = make_ctx(w)
    path, splits = ctx.query_plan(w.batch, w.q_seq, 1, w.width)
    banner(f"capacity step graph: path {path} splits {splits}")
    assert path == 4 and splits > 1
    e = capacity_device(w, inp, ctx=ctx, one_call=True)
    assert e["word"] == 0, e["msg"]
    k0, v0 = tt(inp["past_k"]), tt(inp["past_v"])
    kc, vc = k0.clone(), v0.clone()
    q, ck, cv, ix, bias = tt(inp["q"]), tt(inp["cur_k"]), tt(inp["cur_v"]), tt(inp["indices"]), tt(inp["bias"])
    vl = torch.zeros((w.batch,), dtype=torch.int32, device="cuda")
    wp = torch.zeros_like(vl)
    y = torch.zeros((w.batch, w.hq, w.q_seq, w.dv), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.capacity_step(q, w.batch, w.q_seq, kc, vc, w.cap, ck, cv, w.cur, ix, 1, w.width, bias, y, vl, wp,
                          reset_error=True)
    for rep in range(3):
        y.zero_()
        kc.copy_(k0)  # eager work between replays
        vc.copy_(v0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y_as_f32(y), e["y"]), rep
        assert np.array_equal(to_np(vl), e["valid"]) and np.array_equal(to_np(wp), e["wpos"])
        assert np.array_equal(raw_bytes(to_np(kc)), raw_bytes(e["k"])) and np.array_equal(raw_bytes(to_np(vc)),
                                                                                         raw_bytes(e["v"]))
        assert ctx.read_error()[0] == 0
    ctx.destroy()


LATENT_CAPACITY = {
    "latent_bf16": W.WORKLOADS["decode_bf16"].scaled(batch=3, past=700, topk=500, width=520, capacity=900),
    "latent_bf16_rows": W.WORKLOADS["decode_bf16"].scaled(batch=2, q_seq=3, cur=3, past=300, topk=250,
                                                          width=260, capacity=400, seed=31),
    "fp8_records": W.WORKLOADS["decode_fp8"].scaled(batch=3, past=600, topk=400, width=420, capacity=800),
}


@pytest.mark.parametrize("name", list(LATENT_CAPACITY))
def test_capacity_step_shared_latent(name):
    """sparse_attn_capacity_step over a shared-latent cache (bf16 rows in one
    launch with the lengths; fp8 records through kv_append): lengths, write
    positions and the in-place present bit-exact, Y within tolerance, on the
    shared-latent MFMA kernel of the layout. The bias frontier of batch entry
    b sits at total - b, so the write positions differ from the generator's
    past length; index rows are cut to the recovered length."""
    import torch
    w = LATENT_CAPACITY[name]
    fp8 = w.cache_format == W.CACHE_FP8
    inp = W.make_numpy(w)
    B, cap = w.batch, w.cap
    rng = np.random.default_rng(40)
    b32 = rng.standard_normal((B, 1, w.q_seq, cap)).astype(np.float32)
    for b in range(B):
        b32[b, :, :, w.total - b:] = -np.inf
        b32[b, :, :, rng.integers(0, w.total - b - 1, 5)] = -np.inf  # holes do not move the frontier
    bias = bias_store(b32, w.dtype)
    valid, wpos = oracle.capacity_lengths(bias, cap, w.cur, batch=B, heads=w.hq, q_seq=w.q_seq, bias_dtype=w.dtype)
    assert list(valid) == [w.total - b for b in range(B)]
    idx = inp["indices"].copy()
    for b in range(B):  # keep each row valid against its batch entry's length (sorted: cut the tail)
        row = idx[b]
        row[row >= valid[b]] = -1
        for r in row.reshape(-1, w.width):
            keep = r[r >= 0]
            r[:] = -1
            r[:len(keep)] = keep
    word, _, _, _ = oracle.validate_indices(idx, valid)
    assert word == 0
    past, cur = inp["past_k"], inp["cur_k"]
    if fp8:
        past, cur = oracle_records(past, w), oracle_records(cur, w)
    present = oracle.kv_append(past.copy(), wpos, cur)
    fmt = oracle.FP8_BLOCK64 if fp8 else w.dtype
    ref = oracle.forward(inp["q"], present, None, idx, q_dtype=w.dtype, cache_fmt=fmt, kv_layout=w.layout,
                         hkv=w.hkv, dv=w.dv, rope=w.rope, scale=w.scale, softcap=w.softcap, bias=bias, threads=8)
    banner(f"capacity step shared-latent {name}")
    ctx = make_ctx(w)
    assert ctx.query_plan(B, w.q_seq, 1, w.width)[0] == (3 if fp8 else 2)
    kc = tt(past)
    vl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    wp = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    y = torch.full((B, w.hq, w.q_seq, w.dv), float("nan"), dtype=y_dtype(w), device="cuda")
    ctx.capacity_step(tt(inp["q"]), B, w.q_seq, kc, None, cap, tt(cur), None, w.cur, tt(idx), 1, w.width,
                      tt(bias), y, vl, wp, reset_error=True)
    word, _, msg = ctx.read_error()
    ctx.destroy()
    assert word == 0, msg
    np.testing.assert_array_equal(to_np(vl), valid)
    np.testing.assert_array_equal(to_np(wp), wpos)
    assert np.array_equal(raw_bytes(to_np(kc)), raw_bytes(present))
    check_close(y_as_f32(y), ref, w.dtype, f"capacity step {name}")


@pytest.mark.parametrize("kw", [dict(dtype=W.DT_BF16, dk=128, dv=128, q_seq=1, cur=1, seed=11),  # one launch
                                dict(dk=66, dv=66, seed=13)])                                      # two launches
def test_capacity_step_reset_semantics(kw):
    """Without reset the capacity step adds its bits to an earlier launch's;
    with reset it replaces them, whether the reset rides in the length and
    append launch or is a launch of its own."""
    import torch
    w = W.CAPACITY_WORKLOADS["capacity_small"].scaled(**kw)
    inp = W.make_capacity_numpy(w)
    banner(f"capacity step reset semantics {kw}")
    ctx = make_ctx(w)
    early = inp["indices"].copy()
    r = early[-1, 0, -1]
    r[1], r[2] = r[2], r[1]
    full = torch.full((w.batch,), w.cap, dtype=torch.int32, device="cuda")

    def latch_early():
        ctx.reset_error_async()
        ctx.validate_indices(tt(early), w.batch, 1, w.q_seq, w.width, valid_len=full)
        return ctx.read_error()

    def step(reset):
        kc, vc = tt(inp["past_k"]), tt(inp["past_v"])
        vl = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
        wp = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
        y = torch.zeros((w.batch, w.hq, w.q_seq, w.dv), dtype=y_dtype(w), device="cuda")
        ctx.capacity_step(tt(inp["q"]), w.batch, w.q_seq, kc, vc, w.cap, tt(inp["cur_k"]), tt(inp["cur_v"]), w.cur,
                          tt(inp["indices"]), 1, w.width, tt(inp["bias"]), y, vl, wp, reset_error=reset)
        return ctx.read_error()

    e_word, e_fb, e_msg = latch_early()
    assert e_word == (sa_bits("ORDER") | 512)
    assert step(False) == (e_word, e_fb, e_msg)  # kept
    latch_early()
    w1, fb1, _ = step(True)
    assert w1 == 0 and fb1 == 2 ** 64 - 1         # replaced by a clean launch
    ctx.destroy()


def sa_bits(name):
    import sparse_attention_kv_append_amd as sa
    return getattr(sa, "SA_ERR_" + name)
