"""The bandwidth reference read_sections reads exactly the sections score_paged reads, each
once: the XOR of its per-wavefront words equals the XOR of every 32-bit word of those
sections, computed here on the host."""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_quant_amd as dsa

pytestmark = pytest.mark.gpu


def expected_xor(cache, section_offset, page_stride, section_bytes, bt, seq, num_pages):
    acc = np.uint32(0)
    for q in range(bt.shape[0]):
        nblk = min((max(int(seq[q]), 0) + 63) // 64, bt.shape[1])
        for b in range(nblk):
            pg = int(bt[q, b])
            if 0 <= pg < num_pages:
                s = section_offset + pg * page_stride
                acc ^= np.bitwise_xor.reduce(cache[s:s + section_bytes].view(np.uint32))
    return int(acc)


@pytest.mark.parametrize("fmt,section,stride,offset,nreq,max_blocks", [
    ("mxfp4", 4352, 4352, 0, 3, 9),
    ("mxfp4", 4352, 8192, 3840, 8, 40),
    ("fp8", 8448, 8448, 0, 5, 7),
    ("mxfp4", 4352, 4352, 0, 64, 300),
])
def test_read_sections_reads_each_section_once(fmt, section, stride, offset, nreq, max_blocks):
    rng = np.random.default_rng(nreq * 1000 + max_blocks)
    num_pages = nreq * max_blocks
    nbytes = offset + (num_pages - 1) * stride + section + 16
    cache = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    bt = rng.permutation(num_pages).astype(np.int32).reshape(nreq, max_blocks)
    bt[0, 1] = -1                 # skipped entries: negative and out of range
    bt[nreq - 1, 0] = num_pages + 5
    seq = rng.integers(0, max_blocks * 64 + 200, size=nreq).astype(np.int32)
    seq[0] = max_blocks * 64      # a full request, one past the end, one empty
    seq[1 % nreq] = max_blocks * 64 + 100
    seq[2 % nreq] = 0
    dev = torch.device("cuda")
    out = dsa.read_sections(torch.from_numpy(cache).to(dev), num_pages, stride,
                            torch.from_numpy(bt).to(dev), torch.from_numpy(seq).to(dev), fmt,
                            offset)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)))
    assert got == expected_xor(cache, offset, stride, section, bt, seq, num_pages)
