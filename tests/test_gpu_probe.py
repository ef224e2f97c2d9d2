"""The read-bandwidth probe (include/attn_stream_probe.h) runs to completion
on the GPU through the C ABI and leaves its input untouched."""
import pytest
import torch

import decode_attention_kv_attn_amd as A

pytestmark = pytest.mark.gpu


def test_stream_probe_runs_and_reads_only():
    nbytes = 2 * 2048 * 16384                       # two tiles per workgroup
    buf = torch.arange(nbytes // 4, dtype=torch.int32, device="cuda")
    ref = buf.clone()
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    print(f"[probe] {nbytes} bytes", flush=True)
    A.attn_stream_read_probe(buf, nbytes, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, ref)
