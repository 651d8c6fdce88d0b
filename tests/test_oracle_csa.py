"""Pins for the oracle's CSA ratio-4 selected sink attention.

The compressed-sparse-attention pages (onnx-runtime-ep-cpu / -cuda,
src/kernels/compressed_sparse_attention.rs: `ratio4_attention`, the
`csa_ratio4_sink_attention` kernel, `AttentionBias`) define, per (b, s, h), a
softmax over a dense causal window of current_kv rows plus the selected
583-byte records, with exp(head_sink - max) added to the denominator.

Each pin is fixed independently of the oracle:
  (i)   the whole operation == torch's scaled_dot_product_attention in float64
        over the same keys (records decoded by torch's own float8_e4m3fn and
        bfloat16 types), with the sink as one more key of zero value whose
        additive mask is the sink logit, and the bias as the additive mask;
  (ii)  one candidate: y = v * e^s / (e^s + e^sink) (closed form);
  (iii) the dense window's row sets, read off one-hot rows, for cursor cases
        worked out by hand from the pages' window rule;
  (iv)  a record selected twice weighs twice (closed form); negative indices
        are skipped; an index past the complete records is flagged and
        skipped;
  (v)   a per-head constant bias c is the same as the sink lowered by c;
  (vi)  the cursor and bias-shape checks and the invalid denominator flag.
"""
import numpy as np
import pytest
import torch

import oracle
import sa_workloads as W

D = 512


def torch_decode(rec: np.ndarray) -> torch.Tensor:
    """[..., 583] records -> [..., 512] float64 with torch's fp8/bf16 types:
    7 blocks of [E8M0 scale byte, 64 E4M3FN codes], then 64 little-endian bf16."""
    t = torch.from_numpy(np.ascontiguousarray(rec))
    lead = t.shape[:-1]
    blocks = t[..., :455].reshape(*lead, 7, 65)
    scale = torch.pow(2.0, blocks[..., 0].to(torch.float64) - 127.0)
    codes = blocks[..., 1:].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    nope = (codes * scale[..., None]).reshape(*lead, 448)
    tail = t[..., 455:].clone().view(torch.bfloat16).to(torch.float64)
    return torch.cat([nope, tail], -1)


def pack(rows: np.ndarray) -> np.ndarray:
    B, R = rows.shape[:2]
    return oracle.fp8_pack_rows(rows.reshape(B * R, D), 64).reshape(B, R, 583)


def sdpa_reference(inp, rec, windows, scale, bias_full=None):
    """Expected Y [B, S, H, 512] in float64. windows[s] = the relative current_kv
    rows of query s's dense window; bias_full [B, H, S, Cd + K] or None."""
    q = torch.from_numpy(inp["query"]).double()
    ckv = torch.from_numpy(inp["current_kv"]).double()
    sel = inp["selected"][:, 0]
    sink = torch.from_numpy(inp["sink"]).double()
    dec = torch_decode(rec)
    B, S, H, _ = q.shape
    K = sel.shape[-1]
    y = torch.zeros(B, S, H, D, dtype=torch.float64)
    for b in range(B):
        for s in range(S):
            rows = list(windows[s])
            cd = 128
            keys = [ckv[b, r] for r in rows]
            cand = list(range(len(rows)))
            for j in range(K):
                r = int(sel[b, s, j])
                if r >= 0:
                    keys.append(dec[b, r])
                    cand.append(cd + j)
            k = torch.stack(keys + [torch.zeros(D, dtype=torch.float64)])
            n = k.shape[0]
            mask = torch.zeros(H, n, dtype=torch.float64)
            if bias_full is not None:
                bf = torch.from_numpy(bias_full).double()
                mask[:, :n - 1] = bf[b, :, s, cand]
            mask[:, n - 1] = sink
            out = torch.nn.functional.scaled_dot_product_attention(
                q[b, s][:, None, None, :], k.expand(H, 1, n, D).contiguous(),
                k.expand(H, 1, n, D).contiguous(), attn_mask=mask[:, None, None, :], scale=scale)
            y[b, s] = out[:, 0, 0, :]
    return y.numpy()


@pytest.fixture(scope="module")
def small():
    w = W.CSA_WORKLOADS["csa_small"]
    inp = W.make_csa_numpy(w)
    return w, inp, pack(inp["record_rows"])


# total 300, S 3, Tcur 140: base 160, query 0 at 297; window of query s starts
# at max(160, 297 + s + 1 - 128) = 170 + s, i.e. relative rows 10 + s .. 137 + s
SMALL_WINDOWS = {0: range(10, 138), 1: range(11, 139), 2: range(12, 140)}


def test_sdpa_reference_no_bias(small):
    w, inp, rec = small
    y, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                         inp["sink"], w.total)
    assert flags == 0
    ref = sdpa_reference(inp, rec, SMALL_WINDOWS, 1.0 / np.sqrt(512.0))
    np.testing.assert_allclose(y, ref, atol=1e-5, rtol=0)


def test_sdpa_reference_full_bias_and_scale(small):
    w, inp, rec = small
    rng = np.random.default_rng(5)
    bias = rng.standard_normal((w.batch, w.heads, w.seq, 128 + w.topk)).astype(np.float32)
    y, flags = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                         inp["sink"], w.total, scale=0.03, bias=bias)
    assert flags == 0
    ref = sdpa_reference(inp, rec, SMALL_WINDOWS, float(np.float32(0.03)), bias_full=bias)
    np.testing.assert_allclose(y, ref, atol=1e-5, rtol=0)


def test_single_candidate_closed_form():
    # total 1, one query, one current row: the window is that row alone; no
    # record is complete (total/4 == 0), the selection is all padding
    rng = np.random.default_rng(1)
    H = 4
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    ckv = rng.standard_normal((1, 1, D)).astype(np.float32)
    rec = np.zeros((1, 1, 583), np.uint8)
    sel = np.full((1, 1, 1, 4), -1, np.int32)
    sink = np.array([0.5, -2.0, 3.0, 0.0], np.float32)
    y, flags = oracle.csa_sink_attention(q, ckv, rec, sel, sink, 1)
    assert flags == 0
    v = ckv[0, 0].astype(np.float64)
    s = (q[0, 0].astype(np.float64) @ v) / np.sqrt(512.0)
    w = np.exp(s) / (np.exp(s) + np.exp(sink.astype(np.float64)))
    np.testing.assert_allclose(y[0, 0], w[:, None] * v[None, :], atol=2e-6, rtol=1e-6)


def window_sets(total, S, T, heads=2):
    """Run the oracle with Q = 0 and one-hot current rows; returns, per query,
    the set of relative rows with nonzero weight and the weights."""
    q = np.zeros((1, S, heads, D), np.float32)
    ckv = np.zeros((1, T, D), np.float32)
    for r in range(T):
        ckv[0, r, r] = 1.0
    rec = np.zeros((1, max(1, total // 4), 583), np.uint8)
    sel = np.full((1, 1, S, 1), -1, np.int32)
    sink = np.full(heads, -1e30, np.float32)  # e^(sink - 0) == 0: plain softmax
    y, flags = oracle.csa_sink_attention(q, ckv, rec, sel, sink, total)
    assert flags == 0
    out = []
    for s in range(S):
        nz = np.nonzero(y[0, s, 0])[0]
        out.append((set(int(i) for i in nz), y[0, s, 0, nz]))
        np.testing.assert_array_equal(y[0, s, 0], y[0, s, 1])
    return out


@pytest.mark.parametrize("total,S,T,expect", [
    # prefill from position 0 with 5 rows: query s sees rows 0..s
    (5, 5, 5, {s: set(range(s + 1)) for s in range(5)}),
    # base 70, query at 199: the window starts at max(70, 72) = 72 -> rows 2..129
    (200, 1, 130, {0: set(range(2, 130))}),
    # base 0, queries at 136..139: windows start at 9..12, end at the query
    (140, 4, 140, {0: set(range(9, 137)), 3: set(range(12, 140))}),
    # prefill of 200 from 0: 128 candidates; query 150 sees 23..150, query 10 sees 0..10,
    # query 127 sees 0..127, query 128 sees 1..128
    (200, 200, 200, {150: set(range(23, 151)), 10: set(range(11)), 127: set(range(128)),
                     128: set(range(1, 129))}),
])
def test_window_sets(total, S, T, expect):
    got = window_sets(total, S, T)
    for s, rows in expect.items():
        assert got[s][0] == rows, s
        np.testing.assert_allclose(got[s][1], 1.0 / len(rows), rtol=1e-6)


def records_only_case(sel_row, total=400, T=128, H=2, seed=3):
    """One query; a -inf bias over the 128 window candidates leaves the records."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    ckv = rng.standard_normal((1, T, D)).astype(np.float32)
    rows = W._widen(W._bf16_bits(rng.standard_normal((1, total // 4, D)).astype(np.float32)),
                    W.DT_BF16)
    rec = pack(rows)
    K = len(sel_row)
    sel = np.array(sel_row, np.int32).reshape(1, 1, 1, K)
    bias = np.zeros((1, 1, 1, 128 + K), np.float32)
    bias[..., :128] = -np.inf
    sink = np.array([0.25, -1.0], np.float32)[:H]
    return q, ckv, rec, sel, sink, bias, total


def test_duplicate_record_weighs_twice():
    q, ckv, rec, sel, sink, bias, total = records_only_case([7, 7, -1])
    y, flags = oracle.csa_sink_attention(q, ckv, rec, sel, sink, total, bias=bias)
    assert flags == 0
    v = torch_decode(rec[0, 7]).numpy()
    s = (q[0, 0].astype(np.float64) @ v) / np.sqrt(512.0)
    w = 2 * np.exp(s) / (2 * np.exp(s) + np.exp(sink.astype(np.float64)))
    np.testing.assert_allclose(y[0, 0], w[:, None] * v[None, :], atol=2e-6, rtol=1e-6)


def test_negative_skipped_and_out_of_range_flagged():
    q, ckv, rec, sel, sink, bias, total = records_only_case([5, -1, 30, -7, 99])
    # 100 records are complete (total 400): 99 is valid; now make one index 100
    y_ok, f_ok = oracle.csa_sink_attention(q, ckv, rec, sel, sink, total, bias=bias)
    assert f_ok == 0
    sel_bad = sel.copy()
    sel_bad[0, 0, 0, 2] = 100
    rec_big = np.concatenate([rec, rec[:, :1]], axis=1)  # capacity 101: row 100 exists
    y_bad, f_bad = oracle.csa_sink_attention(q, ckv, rec_big, sel_bad, sink, total, bias=bias)
    assert f_bad == oracle.CSA_RANGE
    sel_skip = sel.copy()
    sel_skip[0, 0, 0, 2] = -1
    y_skip, f_skip = oracle.csa_sink_attention(q, ckv, rec, sel_skip, sink, total, bias=bias)
    assert f_skip == 0
    np.testing.assert_array_equal(y_bad, y_skip)
    # -7 behaves as -1
    sel_m1 = sel.copy()
    sel_m1[0, 0, 0, 3] = -1
    y_m1, _ = oracle.csa_sink_attention(q, ckv, rec, sel_m1, sink, total, bias=bias)
    np.testing.assert_array_equal(y_ok, y_m1)


def test_selection_order_does_not_matter(small):
    w, inp, rec = small
    y, _ = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                     inp["sink"], w.total)
    perm = np.random.default_rng(9).permutation(w.topk)
    y2, _ = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec,
                                      inp["selected"][..., perm], inp["sink"], w.total)
    np.testing.assert_allclose(y, y2, atol=1e-6, rtol=0)


def test_head_bias_equals_lowered_sink(small):
    w, inp, rec = small
    c = np.linspace(-2.0, 2.0, w.heads).astype(np.float32)
    y_b, _ = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                       inp["sink"], w.total, bias=c[:, None, None])
    y_s, _ = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                       (inp["sink"] - c).astype(np.float32), w.total)
    np.testing.assert_allclose(y_b, y_s, atol=2e-6, rtol=0)


def test_index_head_zero_is_read(small):
    w, inp, rec = small
    sel = inp["selected"].copy()
    sel[:, 1:] = 0  # other index heads are not read
    y1, _ = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, inp["selected"],
                                      inp["sink"], w.total)
    y2, _ = oracle.csa_sink_attention(inp["query"], inp["current_kv"], rec, sel, inp["sink"], w.total)
    np.testing.assert_array_equal(y1, y2)


@pytest.mark.parametrize("total,S,T,cap,bias_k", [
    (3, 4, 3, 1, None),        # total < S
    (200, 1, 100, 50, None),   # current_kv starts at 100, the query needs 72
    (200, 1, 130, 49, None),   # 50 complete records, capacity 49
    (200, 1, 130, 50, 129),    # bias last extent neither 1 nor 128 + 2
    (10, 1, 11, 2, None),      # Tcur > total
])
def test_geometry_errors(total, S, T, cap, bias_k):
    q = np.zeros((1, S, 2, D), np.float32)
    ckv = np.zeros((1, T, D), np.float32)
    rec = np.zeros((1, cap, 583), np.uint8)
    sel = np.full((1, 1, S, 2), -1, np.int32)
    bias = None if bias_k is None else np.zeros((1, 1, 1, bias_k), np.float32)
    _, flags = oracle.csa_sink_attention(q, ckv, rec, sel, np.zeros(2, np.float32), total, bias=bias)
    assert flags == oracle.CSA_GEOMETRY


def test_invalid_denominator_flags():
    rng = np.random.default_rng(2)
    q = (rng.standard_normal((1, 1, 2, D)) * 1e-3).astype(np.float32)
    ckv = rng.standard_normal((1, 8, D)).astype(np.float32)
    rec = np.zeros((1, 2, 583), np.uint8)
    sel = np.full((1, 1, 1, 2), -1, np.int32)
    _, f = oracle.csa_sink_attention(q, ckv, rec, sel, np.array([200.0, 0.0], np.float32), 8)
    assert f == oracle.CSA_DENOM  # e^(200 - ~0) overflows fp32
    _, f = oracle.csa_sink_attention(q, ckv, rec, sel, np.array([80.0, 0.0], np.float32), 8)
    assert f == 0
    # one NaN candidate score: max passes over it, the denominator is NaN
    cn = ckv.copy()
    cn[0, 3, 7] = np.nan
    _, f = oracle.csa_sink_attention(q, cn, rec, sel, np.zeros(2, np.float32), 8)
    assert f == oracle.CSA_DENOM
    # every score NaN: no candidate survives the max, the row is zeros, no flag
    qn = q.copy()
    qn[0, 0, 1, 3] = np.nan
    y, f = oracle.csa_sink_attention(qn, ckv, rec, sel, np.zeros(2, np.float32), 8)
    assert f == 0 and not y[0, 0, 1].any()


def test_prefill_from_zero_short_window_candidate_numbering():
    # total == S: the dense candidate count is min(Tcur, 128) = 8, so a bias over
    # [.., 8 + K] is well formed and its entry 8 + j belongs to selected slot j
    rng = np.random.default_rng(4)
    S = T = total = 8
    q = rng.standard_normal((1, S, 2, D)).astype(np.float32)
    ckv = rng.standard_normal((1, T, D)).astype(np.float32)
    rows = W._widen(W._bf16_bits(rng.standard_normal((1, 2, D)).astype(np.float32)), W.DT_BF16)
    rec = pack(rows)
    sel = np.full((1, 1, S, 2), -1, np.int32)
    sel[0, 0, 3:, 0] = 0           # record 0 is complete from position 3
    sel[0, 0, 7:, 1] = 1           # record 1 from position 7
    sink = np.zeros(2, np.float32)
    bias = np.zeros((1, 1, 1, 8 + 2), np.float32)
    bias[..., 8] = -np.inf         # removes selected slot 0
    y_b, f = oracle.csa_sink_attention(q, ckv, rec, sel, sink, total, bias=bias)
    assert f == 0
    sel0 = sel.copy()
    sel0[..., 0] = -1
    y_s, f = oracle.csa_sink_attention(q, ckv, rec, sel0, sink, total)
    assert f == 0
    np.testing.assert_array_equal(y_b, y_s)
    _, f = oracle.csa_sink_attention(q, ckv, rec, sel, sink, total,
                                     bias=np.zeros((1, 1, 1, 128 + 2), np.float32))
    assert f == oracle.CSA_GEOMETRY
