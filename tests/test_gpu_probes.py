"""The library's measurement probes (matrix-core rate, streaming HBM read):
they launch, report their work, and the read probe touches every word of
its buffer (checked through the per-chunk XOR it writes)."""
import numpy as np
import pytest

from block_sparse_causal_amd import stem

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_mfma_probe_reports_work_and_finite_results():
    import torch
    sink = torch.full((4096,), float("nan"), dtype=torch.float32, device="cuda")
    for rnd in (True, False):
        flops = stem.stem_probe_mfma(rnd, sink)
        torch.cuda.synchronize()
        props = torch.cuda.get_device_properties(0)
        # 16 workgroups of 4 wavefronts per CU, 512 trips of 16 products of 32x32x16
        assert flops == props.multi_processor_count * 16 * 4 * 512 * 16 * 32 * 32 * 16 * 2
        n = props.multi_processor_count * 16
        assert torch.isfinite(sink[:n]).all()


def test_mfma_probe_rejects_small_sink():
    import torch
    sink = torch.empty(8, dtype=torch.float32, device="cuda")
    with pytest.raises(stem.StemError):
        stem.stem_probe_mfma(True, sink)


@pytest.mark.parametrize("nwords", [4, 4100, (1 << 22) + 12])
def test_hbm_probe_reads_every_word_once(nwords):
    import torch
    g = torch.Generator().manual_seed(nwords)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nwords,), dtype=torch.int64, generator=g)
    buf = host.to(torch.int32).to("cuda")
    chunks = -(-4 * nwords // 65536)
    sink = torch.zeros(chunks + 3, dtype=torch.int32, device="cuda")
    assert stem.stem_probe_hbm_read(buf, sink) == 4 * nwords
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.to(torch.int32).numpy().view(np.uint32))
    assert got == want


def test_hbm_probe_rejects_bad_sizes():
    import torch
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(stem.StemError):
        stem.stem_probe_hbm_read(torch.zeros(3, dtype=torch.int32, device="cuda"), sink)
    # 65 chunks of 64 KiB need 65 sink words
    with pytest.raises(stem.StemError):
        stem.stem_probe_hbm_read(torch.zeros(65 * 16384, dtype=torch.int32, device="cuda"), sink)
