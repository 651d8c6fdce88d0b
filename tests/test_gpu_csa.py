"""GPU parity of CSA ratio-4 selected sink attention (sparse_attn_csa_forward,
through the C ABI) against the oracle on the same seeded inputs.

Inputs come from sa_workloads' CSA generator; records are made by the oracle's
block quantizer from the generator's bf16 rows and uploaded, so both sides read
the same bytes. The bar is the fp32 one: max |y - y_oracle| <= 1e-5; error
words must match the oracle's flags (range, denominator, geometry).
"""
import numpy as np
import pytest

import oracle
import sa_workloads as W

pytestmark = pytest.mark.gpu

ATOL = 1e-5


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


def pack(rows):
    B, R = rows.shape[:2]
    return oracle.fp8_pack_rows(rows.reshape(B * R, 512), 64).reshape(B, R, 583)


@pytest.fixture(scope="module")
def ctx():
    import sparse_attention_kv_append_amd as sa
    return sa.Context(num_heads=16, kv_num_heads=1, head_dim_qk=64, head_dim_v=64, dtype=sa.SA_F32)


def run_gpu(ctx, inp, rec, total, *, scale=0.0, bias=None, reset=True):
    import torch
    dev = "cuda"
    q = torch.from_numpy(inp["query"]).to(dev)
    ckv = torch.from_numpy(inp["current_kv"]).to(dev)
    r = torch.from_numpy(np.ascontiguousarray(rec)).to(dev)
    sel = torch.from_numpy(np.ascontiguousarray(inp["selected"], np.int32)).to(dev)
    sink = torch.from_numpy(inp["sink"]).to(dev)
    tot = torch.tensor([total], dtype=torch.int64, device=dev)
    y = torch.full(q.shape, 123.0, dtype=torch.float32, device=dev)
    b = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, np.float32)).to(dev)
    if reset:
        ctx.reset_error_async()
    ctx.csa_forward(q, ckv, r, sel, sink, tot, y, scale=scale, bias=b)
    torch.cuda.synchronize()
    word, _, msg = ctx.read_error()
    return y.cpu().numpy(), word, msg


def expect_close(y, ref):
    err = np.abs(y.astype(np.float64) - ref.astype(np.float64))
    assert np.isfinite(y).all()
    assert err.max() <= ATOL, f"max |err| {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"


def case(name="csa_small", **kw):
    w = W.CSA_WORKLOADS[name].scaled(**kw)
    inp = W.make_csa_numpy(w)
    rows = inp["record_rows"]
    cap = w.cap
    if cap > rows.shape[1]:
        pad = np.zeros((w.batch, cap - rows.shape[1], 512), np.float32)
        pad[...] = 7.5
        rows = np.concatenate([rows, pad], axis=1)
    return w, inp, pack(rows)


@pytest.mark.parametrize("kw", [
    dict(),                                                      # S 3, H 32, K 40, Tcur 140
    dict(seq=1, heads=16, topk=96, total=1000, cur_len=300),     # decode, three record tiles
    dict(seq=5, heads=48, topk=33, total=301, cur_len=160, record_cap=90),  # ragged, spare capacity
    dict(batch=3, seq=2, heads=16, topk=2048, total=9000, cur_len=129),     # the widest row
])
def test_csa_matches_oracle(ctx, kw):
    w, inp, rec = case(**kw)
    banner(f"csa {w}")
    ref, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                           inp["sink"], w.total)
    assert flags == 0
    y, word, msg = run_gpu(ctx, inp, rec, w.total)
    assert word == 0, msg
    expect_close(y, ref)


def test_csa_prefill_from_zero(ctx):
    # total == S: the window count is min(Tcur, 128), queries see 1..128 rows,
    # early queries have no complete record (all -1 rows)
    w, inp, rec = case(batch=1, seq=200, heads=16, cur_len=200, total=200, topk=60, index_heads=1)
    banner("csa prefill from position 0, 200 queries")
    ref, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                           inp["sink"], w.total)
    assert flags == 0
    y, word, msg = run_gpu(ctx, inp, rec, w.total)
    assert word == 0, msg
    expect_close(y, ref)


@pytest.mark.parametrize("shape", ["full", "head", "cand", "batch1", "scalar"])
def test_csa_bias_broadcast(ctx, shape):
    w, inp, rec = case()
    C = 128 + w.topk
    rng = np.random.default_rng(11)
    dims = {"full": (w.batch, w.heads, w.seq, C), "head": (w.heads, 1, 1), "cand": (1, 1, 1, C),
            "batch1": (w.batch, 1, 1, 1), "scalar": (1,)}[shape]
    bias = rng.standard_normal(dims).astype(np.float32)
    banner(f"csa bias {dims}")
    ref, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                           inp["sink"], w.total, scale=0.05, bias=bias)
    assert flags == 0
    y, word, msg = run_gpu(ctx, inp, rec, w.total, scale=0.05, bias=bias)
    assert word == 0, msg
    expect_close(y, ref)


def test_csa_out_of_range_record_flagged_and_skipped(ctx):
    import sparse_attention_kv_append_amd as sa
    w, inp, rec = case(record_cap=80)
    inp["selected"][1, 0, 2, 5] = 75  # total 300: records 0..74 are complete
    inp["selected"][0, 0, 0, 0] = -9  # skipped like -1
    banner("csa record index past the complete ones")
    ref, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                           inp["sink"], w.total)
    assert flags == oracle.CSA_RANGE
    y, word, _ = run_gpu(ctx, inp, rec, w.total)
    assert word == sa.SA_ERR_RANGE | sa.SA_ERR_INDEX_ANY
    expect_close(y, ref)


@pytest.mark.parametrize("total,S,T,cap", [
    (2, 3, 2, 1),       # total < S
    (300, 3, 100, 75),  # current_kv starts at 200, query 297 needs 170
    (300, 3, 140, 74),  # 75 complete records, capacity 74
])
def test_csa_geometry_error(ctx, total, S, T, cap):
    import sparse_attention_kv_append_amd as sa
    w, inp, rec = case(seq=S, cur_len=T, total=max(total, 8), topk=4, heads=16)
    inp["selected"][...] = -1
    rec = rec[:, :cap] if rec.shape[1] >= cap else np.zeros((w.batch, cap, 583), np.uint8)
    banner(f"csa geometry total {total} S {S} Tcur {T} cap {cap}")
    _, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                         inp["sink"], total)
    assert flags == oracle.CSA_GEOMETRY
    _, word, _ = run_gpu(ctx, inp, rec, total)
    assert word == sa.SA_ERR_CSA_GEOMETRY


def test_csa_bias_extent_checked_on_device(ctx):
    import sparse_attention_kv_append_amd as sa
    w, inp, rec = case()
    bias = np.zeros((1, 1, 1, 128 + w.topk - 1), np.float32)  # within the host's range, wrong for total
    _, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                         inp["sink"], w.total, bias=bias)
    assert flags == oracle.CSA_GEOMETRY
    _, word, _ = run_gpu(ctx, inp, rec, w.total, bias=bias)
    assert word == sa.SA_ERR_CSA_GEOMETRY


def test_csa_invalid_denominator_flagged(ctx):
    import sparse_attention_kv_append_amd as sa
    w, inp, rec = case()
    inp["current_kv"][0, 100, 9] = np.nan
    _, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                         inp["sink"], w.total)
    assert flags == oracle.CSA_DENOM
    _, word, _ = run_gpu(ctx, inp, rec, w.total)
    assert word == sa.SA_ERR_CSA_DENOM


def test_csa_host_errors(ctx):
    import torch

    import sparse_attention_kv_append_amd as sa
    dev = "cuda"
    q = torch.zeros((1, 1, 24, 512), device=dev)
    ckv = torch.zeros((1, 4, 512), device=dev)
    rec = torch.zeros((1, 2, 583), dtype=torch.uint8, device=dev)
    sel = torch.zeros((1, 1, 1, 4), dtype=torch.int32, device=dev)
    sink = torch.zeros(24, device=dev)
    tot = torch.tensor([4], dtype=torch.int64, device=dev)
    y = torch.zeros_like(q)
    with pytest.raises(sa.SparseAttnError) as e:
        ctx.csa_forward(q, ckv, rec, sel, sink, tot, y)  # 24 heads
    assert e.value.status == sa.SA_E_UNSUPPORTED
    q16 = torch.zeros((1, 1, 16, 512), device=dev)
    with pytest.raises(sa.SparseAttnError) as e:
        ctx.csa_forward(q16, ckv, rec, sel, sink[:16], tot, torch.zeros_like(q16),
                        bias=torch.zeros((2, 1, 1, 1), device=dev))  # batch extent 2 != 1
    assert e.value.status == sa.SA_E_SHAPE


def test_csa_fullsize_decode_sampled_rows():
    """The benchmark's CSA decode workload (batch 64, 64 heads, 16384 records
    per entry, top-512, window 128) in its launch configuration; Y of sampled
    batch entries, all heads, against the oracle run on those entries alone
    (records packed by the oracle's quantizer from the generator's rows)."""
    import torch

    import bench
    banner("csa full-size decode: building inputs")
    s = bench.CsaSetup("csa_decode", 1)
    banner("csa full-size decode: one step")
    s.step(0)
    torch.cuda.synchronize()
    word, _, msg = s.ctx.read_error()
    assert word == 0, msg
    y = s.y.cpu().numpy()
    bs = [0, 5, 40, 63]
    for b, inp in zip(bs, s.oracle_inputs(bs)):
        banner(f"csa full-size decode: oracle on batch entry {b}")
        expect_close(y[b:b + 1], s.oracle_y(inp))
    s.ctx.destroy()
