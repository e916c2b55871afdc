"""Score and select captured into a HIP graph and replayed.

Every call's host tables (the sequence plan) reach the device through
kernel arguments, so tri_score, tri_select_compact and tri_score_noalloc
can be stream-captured: the graph holds only kernel launches (no memset or
host-copy nodes).  Each replay, with eager work on the same buffers between
replays, must reproduce the eager call bit for bit.  The decode-loop driver
may allocate and refuses a capturing stream before queueing anything.
"""
import numpy as np
import pytest
import torch

import rope_aware_key_amd as R
import synth
from harness import pinned, shape_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _buffers(case):
    G, d = case.shape.group, case.shape.head_dim
    rows, out_rows = case.total_rows(), case.total_out_rows()
    return dict(scores=torch.empty(rows, dtype=torch.float32, device=DEV),
                raw=torch.empty(rows, G, dtype=torch.float32, device=DEV),
                kept=torch.empty(out_rows, dtype=torch.int32, device=DEV),
                k_out=torch.empty(out_rows, d, dtype=torch.int16, device=DEV),
                v_out=torch.empty(out_rows, d, dtype=torch.int16, device=DEV),
                pos_out=torch.empty(out_rows, dtype=torch.int32, device=DEV))


def _scramble(b):
    # eager work on the outputs between replays (fill kernels, outside any capture)
    b["scores"].fill_(float("nan"))
    b["raw"].fill_(float("nan"))
    b["kept"].fill_(-7)
    b["k_out"].fill_(3)
    b["v_out"].fill_(5)
    b["pos_out"].fill_(-9)


@pytest.mark.parametrize("noalloc", [False, True])
def test_score_select_graph_replays_match_eager(noalloc):
    case = synth.build_case("graph", synth.Shape(128, 28, 4, 2), [5000, 3001, 64], [512, 256, 100],
                            device=DEV, seed=21)
    sh = shape_of(case)
    cu, cp, bu = (pinned(case.cu_len, np.int64), pinned(case.cur_pos, np.int32),
                  pinned(case.budget, np.int32))
    ws = torch.empty(R.tri_workspace_bytes(sh, cu), dtype=torch.uint8, device=DEV)
    b = _buffers(case)

    def step():
        st = torch.cuda.current_stream()
        args = (sh, cu, cp, case.k, case.k_pos, case.q_centre, case.q_absmean, case.q_R,
                b["scores"])
        if noalloc:
            R.tri_score_noalloc(*args, raw_scores=b["raw"], stream=st)
        else:
            R.tri_score(*args, raw_scores=b["raw"], workspace=ws, stream=st)
        R.tri_select_compact(sh, cu, bu, b["scores"], case.k, case.v, case.k_pos, b["kept"],
                             b["k_out"], b["v_out"], b["pos_out"], workspace=ws, stream=st)

    _scramble(b)
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in b.items()}
    assert torch.isfinite(ref["scores"]).all()

    g = torch.cuda.CUDAGraph()
    _scramble(b)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        _scramble(b)
        g.replay()
        torch.cuda.synchronize()
        for k in b:
            assert torch.equal(b[k], ref[k]), f"replay {rep}: {k}"
        step()   # an eager call between replays, on the same workspace
        torch.cuda.synchronize()
        for k in b:
            assert torch.equal(b[k], ref[k]), f"eager after replay {rep}: {k}"
    print(f"noalloc={noalloc}: 3 replays equal to the eager call", flush=True)


def test_decode_driver_refuses_capture():
    case = synth.build_case("graph_dec", synth.Shape(128, 8, 2, 1), [300], [256], device=DEV, seed=3)
    sh = shape_of(case)
    dec = R.Decode(sh, 1, 256, 128, case.q_centre, case.q_absmean, case.q_R)
    dec.prefill(case.cu_len, case.cur_pos, case.k, case.v, case.k_pos)
    torch.cuda.synchronize()
    d = case.shape.head_dim
    k_new = torch.zeros(2, d, dtype=torch.int16, device=DEV)
    v_new = torch.zeros(2, d, dtype=torch.int16, device=DEV)
    g = torch.cuda.CUDAGraph()
    with pytest.raises(R.TriError, match="UNSUPPORTED"):
        with torch.cuda.graph(g):
            dec.append(k_new, v_new, [300])
    torch.cuda.synchronize()
