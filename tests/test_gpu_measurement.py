"""GPU checks of the measurement aids: kvdec_kernel_timing (events stamped from
each call's main-kernel dispatch) and kvdec_stream_read (the streaming-read
reference)."""
import numpy as np
import pytest
import torch

import kvgen
import long_kv_caches_amd as K
from gpu_util import decode_on_gpu, say

pytestmark = pytest.mark.gpu


def test_kernel_timing_counts_main_launches():
    d = kvgen.dense_small(seed=30)
    say("[timing] three decode calls")
    decode_on_gpu(d)  # warm: plans and code objects loaded
    torch.cuda.synchronize()
    K.kvdec_kernel_timing(True)
    for _ in range(3):
        decode_on_gpu(d)
    torch.cuda.synchronize()
    ms, n = K.kvdec_kernel_timing_read()
    K.kvdec_kernel_timing(False)
    assert n == 3  # the split kernel of each call, not the merge
    assert 0.0 < ms < 1000.0
    # disabled: nothing more is recorded, and enabling again starts from zero
    decode_on_gpu(d)
    K.kvdec_kernel_timing(True)
    assert K.kvdec_kernel_timing_read() == (0.0, 0)
    K.kvdec_kernel_timing(False)


def test_stream_read_reads_every_word():
    # one 16-byte piece whose words fold (XOR) to the kernel's sink value: the
    # thread that reads it writes the sink, so the data was read
    magic = 0x9E3779B9
    src = torch.tensor(np.array([magic, 0, 0, 0], np.uint32).view(np.int32), device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("[stream read] 16 bytes")
    K.kvdec_stream_read(src, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == magic
    # a larger buffer whose words fold to anything else leaves the sink alone
    big = torch.ones(1 << 20, dtype=torch.int32, device="cuda")
    sink.zero_()
    K.kvdec_kernel_timing(True)
    K.kvdec_stream_read(big, sink)
    torch.cuda.synchronize()
    ms, n = K.kvdec_kernel_timing_read()
    K.kvdec_kernel_timing(False)
    assert n == 1 and ms > 0.0
    assert int(sink.item()) == 0
