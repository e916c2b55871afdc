"""The fused score kernel's phase counters (tri_debug_set_phase_buffer).

While a phase buffer is set, tri_score runs a copy of the fused kernel that
adds each phase's core-clock cycles of wave 0 of every work-group to the
buffer.  The copy does the same arithmetic, so its scores, raw scores and
statistics are the plain kernel's bits; every work-group that claimed m
tickets makes m + 1 passes (the last one only finalizes), so the passes
exceed the tickets by at most the grid; turning the hook off restores the
plain kernel and leaves the buffer alone.
"""
import pytest
import torch

import rope_aware_key_amd as R
import synth
from harness import gpu_run

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_phase_counters_same_bits_and_pass_count():
    # 16 units of 32768 keys in 768-key chunks: 43 tickets per unit
    case = synth.workload_case("long_reasoning", device=DEV, S=2, L=2, n=32768, B=2048)
    ref = gpu_run(case, raw=True, stats=True, compact=False)
    buf = torch.zeros(8, dtype=torch.int64, device=DEV)
    prev = R.tri_debug_set_phase_buffer(buf)
    try:
        res = gpu_run(case, raw=True, stats=True, compact=False)
    finally:
        R.tri_debug_set_phase_buffer(None)
    assert prev == 0
    torch.cuda.synchronize()
    for key in ("scores", "raw", "head_stats"):
        assert torch.equal(res[key].view(torch.int8), ref[key].view(torch.int8)), key
    c = buf.cpu().tolist()
    tickets = 16 * 43
    assert tickets < c[7] <= 2 * tickets
    assert all(v >= 0 for v in c[:7])
    assert c[0] > 0 and c[4] >= 0 and sum(c[:7]) > c[0]
    # off again: the plain kernel, the buffer untouched
    again = gpu_run(case, raw=True, stats=True, compact=False)
    torch.cuda.synchronize()
    assert buf.cpu().tolist() == c
    assert torch.equal(again["scores"].view(torch.int8), ref["scores"].view(torch.int8))


def test_phase_buffer_argument_checks():
    with pytest.raises(ValueError):
        R.tri_debug_set_phase_buffer(torch.zeros(8, dtype=torch.int64))      # host memory
    with pytest.raises(ValueError):
        R.tri_debug_set_phase_buffer(torch.zeros(4, dtype=torch.int64, device=DEV))
    assert R.tri_debug_set_phase_buffer(None) == 0
