"""GPU: the diagnostic streaming read (the measured read ceiling of bench.py)
reads every byte once: the XOR of its per-workgroup output words equals the
XOR of the buffer's 32-bit words computed on the host, for a single chunk, a
ragged size and a size of many grid strides."""
import numpy as np
import pytest
import torch

import decoder_attention_rope_amd as gqa
from tests.gpu_common import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, (1 << 20) + 48, 96 << 20])
def test_stream_read_xor(nbytes):
    print(f"[case] diag stream read {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    out = torch.zeros(gqa.GQA_DIAG_READ_BLOCKS, dtype=torch.int32, device=DEV)
    gqa.gqa_diag_stream_read(buf, nbytes, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))
