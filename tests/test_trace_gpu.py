"""Stage timing (fdec_trace_start / fdec_trace_stop) on the GPU: each call records
an event before its first kernel and after each kernel; the intervals are the
kernels' times on the stream; tracing leaves results unchanged."""
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import to_dev
from synth import BF16, cascade_case, paged_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def test_trace_marks_each_kernel_and_changes_nothing():
    case = paged_case(501, 4, 32, 8, 128, [3000, 17, 900, 2048], 16, BF16, extra_pages=2, pad="nan")
    d = to_dev(case)
    ref = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=7)
    torch.cuda.synchronize()
    F.trace_start(64)
    outs = [F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=7)
            for _ in range(3)]
    bal = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"])
    ms, kinds = F.trace_stop()
    # 3 two-kernel calls and a balanced call: (start, map, merge) x 4 -> 11 intervals
    assert kinds == [1, 2, 0, 1, 2, 0, 1, 2, 0, 1, 2]
    assert all(m > 0 for m, k in zip(ms, kinds) if k > 0)
    for o, l in outs:
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1])
    # nothing is recorded once the trace has stopped
    F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=7)
    F.trace_start(8)
    ms2, kinds2 = F.trace_stop()
    assert ms2 == [] and kinds2 == []
    del bal


def test_trace_cascade_kernels(monkeypatch):
    # G = 4, Hkv = 8: prefix and suffix blocks in one launch, then the merge; with
    # FDEC_CASCADE_PATH=two the prefix kernel, the suffix kernel and the merge
    case = cascade_case(502, 8, 32, 8, 128, 1024, 64, suffix_lens=[300, 64, 1000, 5, 700, 256, 128, 900])
    d = to_dev(case)
    for env, want in ((None, [1, 2]), ("two", [1, 2, 3])):
        if env:
            monkeypatch.setenv("FDEC_CASCADE_PATH", env)
        else:
            monkeypatch.delenv("FDEC_CASCADE_PATH", raising=False)
        F.trace_start(16)
        F.cascade_decode(d["q"], d["k"], d["v"], d["page_table"], d["prefix_pages"], case.prefix_len, d["seq_lens"])
        ms, kinds = F.trace_stop()
        assert kinds == want and all(m > 0 for m in ms), f"path {env}: {kinds}"


def test_trace_capacity_bounds_the_events():
    case = paged_case(503, 2, 32, 8, 128, [500, 40], 16, BF16, extra_pages=1)
    d = to_dev(case)
    F.trace_start(4)  # start, map, merge, start: the fourth event is the last
    for _ in range(3):
        F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=3)
    ms, kinds = F.trace_stop()
    assert kinds == [1, 2, 0]
