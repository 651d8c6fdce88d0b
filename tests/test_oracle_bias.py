"""Pins for the oracle's optional attention bias and capacity-mode length
recovery (IndexShare page, onnx-runtime-ep-cuda src/kernels/index_share.rs:
`bias_at`, `index_share_row`, `capacity_write_pos`; the CPU page's
`AttentionBias`).

The bias is additive, rank <= 4, broadcast right-aligned against
[B, Hq, Sq, cache positions] and indexed by the selected key's cache position
(not its slot in the index row). Each pin is fixed independently of the oracle:
  (i)   -inf at a cache position == that key removed from the row, bit for bit
        (so the bias is read at the key's position, not at its slot);
  (ii)  a constant bias leaves Y unchanged up to fp32 rounding (softmax shift);
  (iii) a full-rank random bias == a float64 brute force of
        softmax(softcap(scale q.k) + bias) v over the selected keys;
  (iv)  a broadcast bias == numpy.broadcast_to of it to the full shape, bit for
        bit, for every rank and placement of size-1 axes;
  (v)   a row whose keys are all masked gives zeros;
  (vi)  the recovered valid length and write position == a numpy brute force
        (1 + last column with a finite value over heads and queries).
"""
import numpy as np
import pytest

import oracle
import sa_workloads as W

NEG = np.float32(-np.inf)


def widen(bits, dtype):
    if dtype == W.DT_F32:
        return bits.astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def present(inp):
    kc = oracle.kv_append(inp["past_k"].copy(), inp["past_len"], inp["cur_k"])
    vc = oracle.kv_append(inp["past_v"].copy(), inp["past_len"], inp["cur_v"])
    return kc, vc


def fwd(inp, kc, vc, idx=None, **kw):
    w = inp["workload"]
    return oracle.forward(inp["q"], kc, vc, inp["indices"] if idx is None else idx, q_dtype=w.dtype,
                          cache_fmt=w.dtype, kv_layout=w.layout, hkv=w.hkv, dv=w.dv, scale=w.scale,
                          softcap=w.softcap, **kw)


def tiny(**kw):
    w = W.WORKLOADS["tiny_f32"].scaled(**kw)
    inp = W.make_numpy(w)
    return w, inp, *present(inp)


def drop_keys(idx, dead):
    """Remove the keys in `dead` (per batch) from each row, keep the order,
    pad with -1 on the right."""
    out = np.full_like(idx, -1)
    B, Hi, Sq, Wd = idx.shape
    for b in range(B):
        for h in range(Hi):
            for s in range(Sq):
                row = [k for k in idx[b, h, s] if k != -1 and k not in dead[b]]
                out[b, h, s, :len(row)] = row
    return out


def test_neg_inf_at_a_position_removes_that_key():
    w, inp, kc, vc = tiny(batch=2)
    dead = {0: {3, 17, 40}, 1: {0, 63, 22}}
    bias = np.zeros((w.batch, 1, 1, w.cap), np.float32)
    for b, ks in dead.items():
        bias[b, 0, 0, list(ks)] = NEG
    y = fwd(inp, kc, vc, bias=bias)
    ref = fwd(inp, kc, vc, idx=drop_keys(inp["indices"], dead))
    np.testing.assert_array_equal(y, ref)


def test_constant_bias_is_a_softmax_shift():
    w, inp, kc, vc = tiny()
    y0 = fwd(inp, kc, vc)
    for c in (3.0, -11.5):
        y = fwd(inp, kc, vc, bias=np.array(c, np.float32))
        np.testing.assert_allclose(y, y0, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("softcap", [0.0, 2.5])
def test_full_bias_equals_float64_brute_force(softcap):
    w, inp, kc, vc = tiny(batch=2, softcap=softcap, hq=4, hkv=2)
    rng = np.random.default_rng(7)
    bias = (rng.standard_normal((w.batch, w.hq, w.q_seq, w.cap)) * 2).astype(np.float32)
    bias[rng.random(bias.shape) < 0.2] = NEG
    y = fwd(inp, kc, vc, bias=bias)
    q, k, v = widen(inp["q"], w.dtype), widen(kc, w.dtype), widen(vc, w.dtype)
    idx = inp["indices"]
    group = w.hq // w.hkv
    for b in range(w.batch):
        for h in range(w.hq):
            for s in range(w.q_seq):
                keys = [int(x) for x in idx[b, 0, s] if x != -1]
                kk = k[b, h // group, keys]
                sc = kk @ q[b, h, s] * w.scale
                if softcap:
                    sc = softcap * np.tanh(sc / softcap)
                sc = sc + bias[b, h, s, keys].astype(np.float64)
                if np.isneginf(sc).all():
                    ref = np.zeros(w.dv)
                else:
                    e = np.exp(sc - sc.max())
                    ref = (e / e.sum()) @ v[b, h // group, keys]
                np.testing.assert_allclose(y[b, h, s], ref, rtol=2e-5, atol=2e-6)


@pytest.mark.parametrize("shape", [(64,), (4, 1), (1, 4, 64), (2, 1, 1, 64), (2, 4, 4, 1), (1, 1),
                                   (2, 1, 4, 64)])
def test_broadcast_equals_numpy_broadcast_to(shape):
    w, inp, kc, vc = tiny(batch=2)
    rng = np.random.default_rng(8)
    bias = rng.standard_normal(shape).astype(np.float32)
    full = np.ascontiguousarray(np.broadcast_to(bias, (w.batch, w.hq, w.q_seq, w.cap)))
    np.testing.assert_array_equal(fwd(inp, kc, vc, bias=bias), fwd(inp, kc, vc, bias=full))


def test_bf16_bias_and_broadcast_errors():
    w = W.WORKLOADS["tiny_f32"].scaled(dtype=W.DT_BF16, batch=2)
    inp = W.make_numpy(w)
    kc, vc = present(inp)
    bias = np.zeros((w.batch, 1, 1, w.cap), np.uint16)
    bias[1, 0, 0, [5, 9]] = 0xFF80  # bf16 -inf
    y = fwd(inp, kc, vc, bias=bias)
    ref = fwd(inp, kc, vc, idx=drop_keys(inp["indices"], {0: set(), 1: {5, 9}}))
    np.testing.assert_array_equal(y, ref)
    with pytest.raises(ValueError):
        fwd(inp, kc, vc, bias=np.zeros((3, 1, 1, 1), np.uint16))   # batch extent 3 != 2
    with pytest.raises(ValueError):
        fwd(inp, kc, vc, bias=np.zeros((1, 1, 1, 1, 1), np.uint16))  # rank 5


def test_all_masked_row_gives_zeros():
    w, inp, kc, vc = tiny()
    bias = np.zeros((w.hq, w.q_seq, 1), np.float32)
    bias[2, 1, 0] = NEG   # head 2, query 1: every key
    y = fwd(inp, kc, vc, bias=bias)
    assert not y[0, 2, 1].any()
    assert np.abs(y[0, 2, 0]).sum() > 0 and np.abs(y[0, 1, 1]).sum() > 0


def brute_lengths(bias, B, H, S, keys, cur):
    full = np.broadcast_to(bias, (B, H, S, keys))
    fin = np.isfinite(full).any(axis=(1, 2))             # [B, keys]
    valid = np.array([(np.nonzero(fin[b])[0].max() + 1) if fin[b].any() else 0 for b in range(B)])
    return valid, np.where(valid >= cur, valid - cur, 0)


@pytest.mark.parametrize("shape", [(3, 2, 5, 40), (3, 1, 1, 40), (40,), (3, 2, 1, 40), (1, 1, 5, 40)])
def test_capacity_lengths_equal_brute_force(shape):
    rng = np.random.default_rng(9)
    bias = rng.standard_normal(shape).astype(np.float32)
    # a padding frontier per leading entry, with holes and NaN before it
    lead = bias.reshape(-1, shape[-1])
    for i in range(lead.shape[0]):
        f = int(rng.integers(0, shape[-1] + 1))
        lead[i, f:] = NEG
        lead[i, rng.integers(0, shape[-1], 3)] = np.nan
        lead[i, rng.integers(0, shape[-1], 2)] = NEG
    B, H, S, K = 3, 2, 5, 40
    for cur in (1, 4, 45):
        valid, wpos = oracle.capacity_lengths(bias, K, cur, batch=B, heads=H, q_seq=S)
        bv, bw = brute_lengths(bias, B, H, S, K, cur)
        np.testing.assert_array_equal(valid, bv)
        np.testing.assert_array_equal(wpos, bw)


def test_capacity_lengths_special_cases():
    K = 16
    bias = np.full((2, 1, 1, K), NEG)
    bias[0, 0, 0, :9] = 0.0            # causal/padding frontier at 9
    valid, wpos = oracle.capacity_lengths(bias, K, 1, batch=2, heads=3, q_seq=1)
    assert list(valid) == [9, 0] and list(wpos) == [8, 0]
    bias[1, 0, 0, K - 1] = -1e30       # finite at the last column: the whole capacity
    valid, wpos = oracle.capacity_lengths(bias, K, 2, batch=2, heads=3, q_seq=1)
    assert list(valid) == [9, K] and list(wpos) == [7, K - 2]
    bits = np.full((1, K), 0xFF80, np.uint16)   # bf16 -inf, then +inf is not finite either
    bits[0, 3] = 0x7F80
    bits[0, 5] = 0x3F80                          # 1.0
    valid, wpos = oracle.capacity_lengths(bits, K, 1, batch=2, heads=1, q_seq=1, bias_dtype=W.DT_BF16)
    assert list(valid) == [6, 6] and list(wpos) == [5, 5]
