"""The measurement aids behind the bench's re-measured peaks: the streaming
copy must copy every byte (and nothing past the end), the matrix-core loop
must write finite values to every output, and both reject bad arguments on
the host."""
import pytest

import sparse_attention_kv_append_amd as sa

pytestmark = pytest.mark.gpu


def ctx():
    return sa.Context(num_heads=16, kv_num_heads=1, head_dim_qk=64, head_dim_v=64, dtype=sa.SA_F32)


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 1001])
def test_measure_copy_copies_exactly(nbytes):
    import torch
    print(f"\n[gpu] measure_copy {nbytes} bytes", flush=True)
    c = ctx()
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8, device="cuda")
    dst = torch.full((nbytes + 256,), 0xA5, dtype=torch.uint8, device="cuda")
    c.measure_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())
    c.destroy()


def test_measure_read_writes_every_sink_word():
    import torch
    print("\n[gpu] measure_read", flush=True)
    c = ctx()
    n = (32 << 20) + 16 * 77  # enough vectors for every workgroup of the probe
    src = torch.full((n,), 0x11, dtype=torch.uint8, device="cuda")
    sink = torch.full((sa.SA_PEAK_READ_SINK_WORDS + 64,), -7, dtype=torch.int32, device="cuda")
    c.measure_read(sink, src, n)
    torch.cuda.synchronize()
    # each word is the xor of an even or odd number of 0x11111111 words
    assert bool(((sink[:-64] == 0) | (sink[:-64] == 0x11111111)).all())
    assert bool((sink[-64:] == -7).all())
    c.destroy()


def test_measure_mfma_writes_every_output():
    import torch
    print("\n[gpu] measure_mfma 300 workgroups", flush=True)
    c = ctx()
    out = torch.full((300 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    c.measure_mfma(out, 300, 16)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    c.destroy()


def test_measure_host_errors():
    import torch
    c = ctx()
    a = torch.empty(1024, dtype=torch.uint8, device="cuda")
    b = torch.empty(1024, dtype=torch.uint8, device="cuda")
    for call in (lambda: c.measure_copy(a, b, 0), lambda: c.measure_copy(a, b, 24),
                 lambda: c.measure_copy(a[1:], b, 16), lambda: c.measure_copy(a[16:], a, 64),
                 lambda: c.measure_read(torch.empty(16, dtype=torch.int32, device="cuda"), a[8:], 64),
                 lambda: c.measure_read(None, a, 64),
                 lambda: c.measure_mfma(torch.empty(256, device="cuda"), 0, 1),
                 lambda: c.measure_mfma(torch.empty(256, device="cuda"), 1, 0)):
        with pytest.raises(sa.SparseAttnError) as e:
            call()
        assert e.value.status == 1
    c.destroy()
