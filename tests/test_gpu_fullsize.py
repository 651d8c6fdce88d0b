"""GPU parity at the full benchmark sizes, in the launch configuration the
benchmark times (its Setup: same context limits, split count, in-place append
and fused validation in one step).

The oracle cannot run whole full-size steps in seconds, so each test checks:
  * the error word is clean after the step;
  * the present cache bit for bit: appended rows equal the current rows (for
    fp8 records, the oracle quantizer's records of them), every other row is
    unchanged;
  * for fp8, the device's quantize-on-append records of the sampled rows'
    selected keys equal the oracle quantizer's records of the same bf16 rows;
  * Y of sampled (batch, query) rows, all heads, against the oracle run on
    those rows alone (inputs drawn again from the seeded generators, never
    read from what the library wrote), to the bf16 tolerance.
"""
import numpy as np
import pytest

import oracle
import sa_workloads as W
from gpu_support import check_close

pytestmark = pytest.mark.gpu

SAMPLES = {
    "decode_bf16": [(0, 0), (1, 0), (17, 0), (31, 0)],
    "decode_fp8": [(0, 0), (5, 0), (40, 0), (63, 0)],
    "prefill_bf16": [(0, 0), (0, 1), (0, 2046), (0, 2047), (0, 2048), (0, 3001), (0, 4095)],
    "dense_gqa": [(0, 0), (3, 64), (7, 127)],
    "gqa_decode_b2": [(0, 0), (1, 0)],
    # 29700 query rows: past the eight-wave kernel's addressing, so the
    # four-wave kernel runs; rows at both ends and at the limit
    "prefill_long_q": [(0, 0), (0, 15), (0, 29589), (0, 29699)],
}


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)


@pytest.mark.parametrize("name", list(SAMPLES))
def test_fullsize_step_matches_oracle_on_sampled_rows(name):
    import torch

    import bench
    banner(f"full-size {name}: building inputs")
    s = bench.Setup(name, 1)
    w = s.w
    before_k = s.k.clone()
    before_v = None if s.v is None else s.v.clone()
    banner(f"full-size {name}: one step (path {s.path}, splits {s.splits})")
    s.step(0)
    torch.cuda.synchronize()
    word, _, msg = s.ctx.read_error()
    assert word == 0, msg
    assert torch.equal(s.vlen, torch.full_like(s.vlen, w.total))

    # present: rows outside [past, past + cur) untouched, new rows = current rows
    P, C = w.past, w.cur
    for after, before in ((s.k, before_k), (s.v, before_v)):
        if after is None:
            continue
        assert torch.equal(after[:, :, :P], before[:, :, :P])
        assert torch.equal(after[:, :, P + C:], before[:, :, P + C:])
    if s.fp8:
        cur_bits = s.cur_k.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        want = oracle.fp8_pack_rows((cur_bits.astype(np.uint32) << 16).view(np.float32), w.rope)
        assert np.array_equal(s.k[:, :, P:P + C].cpu().numpy(), want)
    else:
        assert torch.equal(s.k[:, :, P:P + C].view(torch.int16), s.cur_k.view(torch.int16))
        if s.v is not None:
            assert torch.equal(s.v[:, :, P:P + C].view(torch.int16), s.cur_v.view(torch.int16))

    rows = SAMPLES[name]
    banner(f"full-size {name}: oracle on rows {rows}")
    inputs = bench.oracle_row_inputs(s, rows)
    y = s.y.float().cpu().numpy()
    worst = 0.0
    for (b, qi), inp in zip(rows, inputs):
        if s.fp8:
            sel = s.idx_host[0][b, 0, qi]
            sel = torch.from_numpy(sel[sel >= 0].astype(np.int64)).cuda()
            dev_rec = s.k[b, 0].index_select(0, sel).cpu().numpy()
            assert np.array_equal(dev_rec, inp["k"]), f"records of row {(b, qi)}"
        ref = bench.oracle_row(s, inp, threads=8)
        worst = max(worst, check_close(y[b, :, qi], ref, W.DT_BF16, f"{name} row {(b, qi)}"))
    banner(f"full-size {name}: max |Y - oracle| over sampled rows = {worst:.3e}")
    s.ctx.destroy()


def test_fullsize_tiny_config_is_whole():
    """The tiny fp32 workload is small enough for the whole step: every row."""
    from gpu_support import check_present, run_device, run_oracle
    w = W.WORKLOADS["tiny_f32"]
    inp = W.make_numpy(w)
    dev = run_device(w, inp)
    assert dev["word"] == 0, dev["msg"]
    y_ref, pk, pv = run_oracle(w, inp)
    check_present(w, dev, pk, pv)
    check_close(dev["y"], y_ref, W.DT_F32, "tiny_f32")
