"""Forward launches with fused validation over index rows holding planted
violations: the error word, the first failing (row, column) and the message
equal the oracle validator's verdict, on every forward path. The generic and
grouped-query paths run the standalone validation kernel before their
forward (the grouped-query kernel validates in its launch only inside the
one-launch step, which tests/test_gpu_step_kv.py covers); the shared-latent
paths validate inside the attention kernels, each workgroup its own columns.

Y of such a launch is not compared (the caller discards it): the launch only
has to stay in bounds and finish. Rows wider than one 2048-key stage of a
workgroup and rows holding only padding are included, since both change how
a workgroup walks its columns."""
import numpy as np
import pytest

import oracle
import sa_workloads as W
from gpu_support import make_ctx, tt

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


def plant_violations(idx, bound, seed, cols=None):
    """Copy of the valid rows `idx` [B, 1, Sq, W] with one planted violation
    in most rows. Columns near each row's end are favoured. With cols =
    (lo, hi) every violation lies in columns [lo, hi) (rows with no such
    column stay valid), so a workgroup that skipped those columns would
    report none of them."""
    rng = np.random.default_rng(seed)
    out = idx.astype(np.int64).copy()
    B, Hi, Sq, Wd = out.shape
    rows = out.reshape(-1, Wd)
    lo_c, hi_c = cols if cols is not None else (0, Wd)
    for r in range(rows.shape[0]):
        T = int(bound[r // (Hi * Sq)])
        n = int((rows[r] >= 0).sum())
        kind = int(rng.integers(0, 8 if cols is None else 6))
        lo = max(0, n - 80) if rng.random() < 0.7 else 0
        lo, hi = max(lo, lo_c), min(n, hi_c)
        if kind == 2:  # a value after the padding: needs a padding column in range
            plo, phi = max(n, lo_c), min(Wd, hi_c)
            if plo < phi:
                rows[r, int(rng.integers(plo, phi))] = int(rng.integers(0, T))
            continue
        if lo >= hi:
            continue
        c = int(rng.integers(lo, hi))
        if kind == 1:
            rows[r, c] = -int(rng.integers(2, 9))                  # sentinel
        elif kind == 3:
            rows[r, c] = T + int(rng.integers(0, 5))                # range
        elif kind == 4 and c >= 1:
            rows[r, c] = rows[r, c - 1]                              # duplicate
        elif kind == 5 and c >= 1:
            rows[r, c - 1], rows[r, c] = rows[r, c], rows[r, c - 1]  # order
        elif kind == 6:
            rows[r, :] = -1                                          # all padding
    return out


PREFILL = W.WORKLOADS["prefill_bf16"]
FP8 = W.WORKLOADS["decode_fp8"]
# rows of 4001 + q keys (q < 128) over width 4200 split in two workgroups of
# 2112 and 2088 columns: each workgroup walks two stages
LATENT_WIDE = PREFILL.scaled(q_seq=128, cur=128, past=4100, width=4200, topk=4200)
# one workgroup per row over 2100 columns: two stages
ONE_WG_WIDE = PREFILL.scaled(q_seq=260, cur=260, past=2000, width=2100, topk=2100)

CASES = {
    # name: (workload, expected plan path, planting seed, planted column range)
    "latent_split": (W.WORKLOADS["decode_bf16"].scaled(batch=12, past=1500, topk=700, width=710), 2, 11, None),
    "latent_wide_first_wg_late": (LATENT_WIDE, 2, 12, (2048, 2112)),
    "latent_wide_second_wg_late": (LATENT_WIDE, 2, 13, (4160, 4200)),
    "latent_one_wg_wide": (ONE_WG_WIDE, 2, 14, None),
    "latent_one_wg_wide_late": (ONE_WG_WIDE, 2, 15, (2048, 2100)),
    "pair_fp8_split": (FP8.scaled(batch=12, past=1200, topk=650, width=650), 3, 16, None),
    "pair_fp8_wide_late": (FP8.scaled(batch=1, q_seq=260, cur=260, past=2000, width=2100, topk=2100,
                                      pattern="causal_prefill"), 3, 17, (2048, 2100)),
    "gqa": (W.WORKLOADS["dense_gqa"].scaled(batch=2, hq=8, hkv=2, q_seq=12, past=500, cur=12,
                                            width=520, topk=520), 4, 18, None),
    # decode rows split over 6 workgroups per (batch, kv head), eight kv heads
    "gqa_split_decode": (W.WORKLOADS["dense_gqa"].scaled(batch=6, hq=32, hkv=8, q_seq=1, past=5000, cur=1,
                                                         width=4000, topk=3900, pattern="uniform",
                                                         softcap=0.0), 4, 20, None),
    "gqa_split_decode_late": (W.WORKLOADS["dense_gqa"].scaled(batch=6, hq=32, hkv=8, q_seq=1, past=5000, cur=1,
                                                              width=4000, topk=3990, pattern="uniform",
                                                              softcap=0.0), 4, 21, (3700, 4000)),
    # one kv head per query head (32 queries per workgroup), three query blocks
    "gqa_group1": (W.WORKLOADS["dense_gqa"].scaled(batch=2, hq=4, hkv=4, q_seq=70, past=300, cur=70,
                                                   width=380, topk=380), 4, 22, None),
    "generic": (W.WORKLOADS["dense_gqa"].scaled(batch=2, hq=8, hkv=2, q_seq=12, past=500, cur=12,
                                                width=520, topk=520, dtype=W.DT_F16), 0, 19, None),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("i64", [False, True])
def test_fused_verdict_matches_oracle(name, i64):
    import torch
    w, path, seed, cols = CASES[name]
    banner(f"fused verdict {name} i64={i64}")
    B, Sq, Wd = w.batch, w.q_seq, w.width
    bound = np.full(B, w.total, np.int32)
    rng = np.random.default_rng(seed)
    idx = plant_violations(W.index_rows(w, rng), bound, seed + 100 * i64, cols)
    if not i64:
        idx = idx.astype(np.int32)
    word, _, first, msg = oracle.validate_indices(idx, bound)
    assert word != 0  # the planting produced violations

    ctx = make_ctx(w, idx64=i64)
    assert ctx.query_plan(B, Sq, 1, Wd)[0] == path
    gen = torch.Generator(device="cuda").manual_seed(seed)
    if w.cache_format == W.CACHE_FP8:
        # any bytes make valid-shaped records: NaN scale / code bytes are
        # avoided so the launch computes finite values (Y is not compared)
        cache = torch.randint(0, 120, (B, 1, w.cap, w.dk + 72), dtype=torch.uint8, device="cuda",
                              generator=gen)
        vcache = None
    else:
        dt = {W.DT_BF16: torch.bfloat16, W.DT_F16: torch.float16, W.DT_F32: torch.float32}[w.dtype]
        cache = torch.randn((B, w.hkv, w.cap, w.dk), device="cuda", generator=gen).to(dt)
        vcache = None if w.layout == W.LAYOUT_SHARED_LATENT else \
            torch.randn((B, w.hkv, w.cap, w.dv), device="cuda", generator=gen).to(dt)
    qdt = {W.DT_BF16: torch.bfloat16, W.DT_F16: torch.float16, W.DT_F32: torch.float32}[w.dtype]
    q = torch.randn((B, w.hq, Sq, w.dk), device="cuda", generator=gen).to(qdt)
    y = torch.empty((B, w.hq, Sq, w.dv), dtype=qdt, device="cuda")
    vlen = tt(bound)
    for rep in range(2):  # the per-row slots re-arm: a second launch gives the same verdict
        ctx.reset_error_async()
        ctx.forward(q, B, Sq, cache, vcache, w.cap, vlen, tt(idx), 1, Wd, y, fused_validate=True)
        dword, dfirst, dmsg = ctx.read_error()
        assert dword == word, f"launch {rep}: word {dword:#x} != {word:#x}"
        assert dfirst == first[0] * (Wd + 1) + first[1], f"launch {rep}"
        assert dmsg == msg
    ctx.destroy()
