"""The HBM read probe (a measurement aid): both access modes run on a small
buffer and report success, and every workgroup writes its sink word (a
buffer of one repeated word XORs to 0 over each 16-byte load)."""
import pytest
import torch

from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunk", [0, 2048])
def test_read_probe_runs(gpu, chunk):
    log(f"read probe chunk {chunk}")
    buf = torch.full((1 << 20,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")   # 4 MiB
    sink = torch.full((gpu.hbm_read_probe_sink_words(),), -1, dtype=torch.int32, device="cuda")
    gpu.hbm_read_probe(buf, chunk, sink)
    torch.cuda.synchronize()
    vals = set(sink.cpu().tolist())
    assert vals == {0}, vals   # every word overwritten from its initial -1
