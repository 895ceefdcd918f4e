"""GPU check of the streaming-read measurement aid (mqa_read_probe): it reads
every word it is given (the sink is written exactly when the XOR of the
buffer's 32-bit words is the documented value) and writes nothing else."""
import pytest
import torch

from gpu_util import announce

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import query_decode_attention_amd as mqa


@pytest.mark.parametrize("words", [4, 4 * 1000 + 4, 4 * (1 << 20)])
def test_read_probe_reads_everything_and_writes_only_the_sink(words):
    announce(f"read probe over {words * 4} bytes")
    buf = torch.zeros(words, dtype=torch.int32, device="cuda")
    sink = torch.zeros(2, dtype=torch.int32, device="cuda")
    mqa.read_probe(buf, sink[:1])
    torch.cuda.synchronize()
    assert sink.tolist() == [0, 0]
    # one word anywhere (here the last one) makes the XOR the documented value
    buf[-4] = 0x5A5AA5A5
    mqa.read_probe(buf, sink[:1])
    torch.cuda.synchronize()
    assert sink.tolist() == [1, 0]
    assert int(buf.count_nonzero()) == 1
