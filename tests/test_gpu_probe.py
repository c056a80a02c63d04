"""GPU check of the read-bandwidth probe behind the bench's measured ceiling:
it must read every 16-byte chunk of the buffer exactly once (an XOR of the
words read, against the same XOR on the host), or the ceiling it reports
would not be a read of the whole buffer."""
import numpy as np
import pytest
import torch

from medusa_tree_attention_attn_amd._lib import tree_attn_stream_read

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 8 + 48, 3 << 20, (5 << 20) + 16 * 37])
def test_stream_read_reads_each_chunk_once(nbytes):
    """Whole 32 KB workgroup iterations, a remainder of 16-byte chunks, and a
    buffer smaller than one iteration; the bytes past the last whole 16-byte
    chunk are not read."""
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2**32, size=nbytes // 4 + 3, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    print(f"stream_read {nbytes} bytes", flush=True)
    tree_attn_stream_read(src, sink, nbytes)
    torch.cuda.synchronize()
    n_words = nbytes // 16 * 4
    want = np.bitwise_xor.reduce(words[:n_words]) if n_words else np.uint32(0)
    assert np.uint32(sink.cpu().numpy()[0]) == np.uint32(want)
