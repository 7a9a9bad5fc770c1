"""The ceiling kernels (benchmark instrumentation).  The streaming read reads every 16-byte
word, ragged tails included, and writes its sink only when the XOR of all words is the fixed
word; the matrix-rate kernel runs in each operand mode without touching its sink."""
import sys

import numpy as np
import pytest
import torch

import lossless_draft_verification_row_amd as L

pytestmark = pytest.mark.gpu
MAGIC = 0x9E3779B9


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("words", [1, 255, 4096, 4097, 6 * 4096 * 1024 + 17])
@pytest.mark.parametrize("where", ["first", "last"])
def test_stream_read_sees_every_word(words, where):
    note(f"case stream_read words={words} where={where}")
    host = np.zeros(words * 4, dtype=np.uint32)
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    L.spec_stream_read(buf, sink)          # all zero: the XOR is 0, the sink keeps its value
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
    host[0 if where == "first" else 4 * words - 1] = MAGIC
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    L.spec_stream_read(buf, sink)          # one word carries the pattern: the sink is written
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MAGIC


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_mfma_rate_runs_and_leaves_the_sink(mode):
    """The matrix-rate kernel runs in every operand mode; its sum is never exactly 2^127, so the
    sink keeps the value it had."""
    note(f"case mfma_rate mode={mode}")
    sink = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    L.spec_mfma_rate(mode, 16, 8, sink)
    torch.cuda.synchronize()
    assert sink.item() == 7.0
