"""The streaming-read measurement helper on the GPU: it reads the buffer and
leaves the sink untouched for data without its marker pattern (here every
16-byte word folds to zero), for sizes with and without a partial last wave."""
import pytest
import torch

import compressed_decode_attention_amd as kvc

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (64 << 20) + 48])
def test_stream_read_runs_and_writes_nothing(nbytes):
    buf = torch.ones(((64 << 20) + 64) // 4, dtype=torch.float32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    kvc.stream_read(buf, sink, nbytes)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
