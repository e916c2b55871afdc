"""C-ABI contract checks that need no GPU: the library loads, exports every
symbol the header declares, and rejects bad arguments before queueing any
device work (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "triattn.h")

R = pytest.importorskip("rope_aware_key_amd", reason="libtriattn.so not built")

ST = {"OK": 0, "INVALID": 1, "UNSUPPORTED": 2, "WORKSPACE": 3, "HIP": 4}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tri_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = ctypes.CDLL(R.LIB_PATH)
    names = declared_functions()
    assert set(names) == {"tri_calibrate", "tri_calibrate_workspace_bytes", "tri_workspace_bytes", "tri_score",
                          "tri_select_compact", "tri_status_string", "tri_last_error",
                          "tri_workspace_bytes_offsets", "tri_score_offsets",
                          "tri_decode_create", "tri_decode_prefill", "tri_decode_append",
                          "tri_decode_get_view", "tri_decode_destroy",
                          "tri_trig_correlation_workspace_bytes", "tri_trig_correlation",
                          "tri_pyramid_budgets", "tri_workspace_bytes_layers",
                          "tri_select_compact_layers", "tri_score_paged",
                          "tri_select_compact_paged", "tri_workspace_bytes_paged",
                          "tri_debug_set_wait_limit", "tri_stream_probe",
                          "tri_score_noalloc", "tri_score_status",
                          "tri_debug_set_resident_groups", "tri_debug_set_phase_buffer"}
    for name in names:
        assert hasattr(lib, name), name
    assert set(R.EXPORTS) == set(names)


def test_status_strings():
    assert R.status_string(0) == "TRI_OK"
    assert R.status_string(3) == "TRI_ERR_WORKSPACE"


FAKE = 0x10000  # never dereferenced: every call below fails validation first


class _Fake:
    def __init__(self, addr=FAKE):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _score(shape, cu, cp, **kw):
    args = dict(k=_Fake(), k_pos=None, q_centre=_Fake(), q_absmean=_Fake(), q_R=_Fake(),
                scores=_Fake(), workspace=None, workspace_bytes=0)
    args.update(kw)
    return R.tri_score(shape, cu, cp, args["k"], args["k_pos"], args["q_centre"],
                       args["q_absmean"], args["q_R"], args["scores"],
                       workspace=args["workspace"], workspace_bytes=args["workspace_bytes"],
                       stream=0)


def _status(fn, *a, **kw):
    try:
        fn(*a, **kw)
        return 0
    except R.TriError as e:
        return e.status


@pytest.mark.parametrize("d,hq,hkv,L,theta,expect", [
    (127, 4, 4, 1, 1e4, "INVALID"), (0, 4, 4, 1, 1e4, "INVALID"), (260, 4, 4, 1, 1e4, "INVALID"),
    (12, 4, 4, 1, 1e4, "INVALID"), (128, 6, 4, 1, 1e4, "INVALID"), (128, 34, 2, 1, 1e4, "UNSUPPORTED"),
    (128, 4, 4, 0, 1e4, "INVALID"), (128, 4, 4, 1, 0.0, "INVALID"), (128, 4, 0, 1, 1e4, "INVALID"),
])
def test_shape_validation(d, hq, hkv, L, theta, expect):
    sh = R.make_shape(d, hq, hkv, L, theta)
    assert _status(_score, sh, [0, 8], [8]) == ST[expect]
    assert R.tri_workspace_bytes(sh, [0, 8]) == 0


def test_score_argument_checks():
    sh = R.make_shape(128, 8, 2, 2)
    cu = [0, 100, 250]
    need = R.tri_workspace_bytes(sh, cu)
    assert need > 0
    assert _status(_score, sh, [0, 100, 90], [1, 2]) == ST["INVALID"]          # decreasing
    assert _status(_score, sh, cu, None) == ST["INVALID"]                      # no cur_pos
    assert _status(_score, sh, cu, [1, 2], k=None) == ST["INVALID"]
    assert _status(_score, sh, cu, [1, 2], scores=None) == ST["INVALID"]
    assert _status(_score, sh, cu, [1, 2], k=_Fake(FAKE + 2)) == ST["INVALID"]  # misaligned
    assert _status(_score, sh, cu, [1, 2], workspace=_Fake(), workspace_bytes=need - 1) == ST["WORKSPACE"]
    assert _status(_score, sh, cu, [1, 2]) == ST["WORKSPACE"]
    # an empty batch queues nothing and succeeds
    assert _status(_score, sh, [0, 0, 0], [1, 2]) == 0
    assert _status(_score, sh, [0], []) == 0                                   # no sequences
    assert _status(_score, sh, [], []) == ST["INVALID"]                        # num_seqs = -1
    assert "num_seqs" in R.last_error()


def _sel(shape, cu, budget, **kw):
    args = dict(scores=_Fake(), k=_Fake(), v=_Fake(), k_pos=_Fake(), kept=_Fake(),
                k_out=_Fake(FAKE * 2), v_out=_Fake(FAKE * 3), pos_out=_Fake(FAKE * 4),
                workspace=None, workspace_bytes=0)
    args.update(kw)
    return R.tri_select_compact(shape, cu, budget, args["scores"], args["k"], args["v"],
                                args["k_pos"], args["kept"], args["k_out"], args["v_out"],
                                args["pos_out"], workspace=args["workspace"],
                                workspace_bytes=args["workspace_bytes"], stream=0)


def test_select_argument_checks():
    sh = R.make_shape(64, 4, 2, 1)
    cu = [0, 50, 80]
    assert _status(_sel, sh, cu, [10, -1]) == ST["INVALID"]
    assert _status(_sel, sh, cu, None) == ST["INVALID"]
    assert _status(_sel, sh, cu, [10, 10], v_out=None) == ST["INVALID"]          # unpaired
    assert _status(_sel, sh, cu, [10, 10], kept=None) == ST["INVALID"]
    assert _status(_sel, sh, cu, [10, 10], k=_Fake(FAKE + 8)) == ST["INVALID"]   # misaligned
    assert _status(_sel, sh, cu, [10, 10]) == ST["WORKSPACE"]
    assert _status(_sel, sh, cu, [0, 0]) == 0                                    # nothing kept
    assert _status(_sel, sh, [0, 0, 0], [5, 5]) == 0


def test_calibrate_argument_checks():
    sh = R.make_shape(64, 4, 2, 1)

    need = R.tri_calibrate_workspace_bytes(sh, 10)
    assert need > 0 and R.tri_calibrate_workspace_bytes(sh, 0) == 0

    def cal(q=_Fake(), n=10, c=_Fake(), a=_Fake(), r=_Fake(), ws=_Fake(), wsb=None):
        return R.tri_calibrate(sh, q, None, n, c, a, r, workspace=ws,
                               workspace_bytes=need if wsb is None else wsb, stream=0)

    assert _status(cal, n=0) == ST["INVALID"]
    assert _status(cal, q=None) == ST["INVALID"]
    assert _status(cal, r=None) == ST["INVALID"]
    assert _status(cal, q=_Fake(FAKE + 2)) == ST["INVALID"]
    assert _status(cal, q=_Fake(FAKE + 8)) == ST["INVALID"]
    assert _status(cal, ws=None, wsb=0) == ST["WORKSPACE"]
    assert _status(cal, wsb=need - 1) == ST["WORKSPACE"]
    assert _status(cal, ws=_Fake(FAKE + 8)) == ST["INVALID"]


def test_wait_limit_hook_round_trip():
    """The test hook swaps the fused kernel's wait bound on the host side
    only (no device work) and hands back the previous value."""
    prev = R.tri_debug_set_wait_limit(7)
    try:
        assert prev == 1 << 22
        assert R.tri_debug_set_wait_limit(9) == 7
    finally:
        R.tri_debug_set_wait_limit(prev)
    assert R.tri_debug_set_wait_limit(prev) == prev


def test_split_select_workspace():
    """Units past 35840 keys take the split select, whose per-tile histograms
    (1 KB per 4096-key tile) and counts are part of the workspace."""
    sh = R.make_shape(64, 2, 2, 3)
    a = R.tri_workspace_bytes_layers(sh, [0, 35840])
    b = R.tri_workspace_bytes_layers(sh, [0, 35841])
    units, tiles = 3 * 2, 9
    assert b - a >= units * tiles * (1024 + 8)


def test_workspace_grows_with_batch():
    sh = R.make_shape(128, 28, 4, 28)
    small = R.tri_workspace_bytes(sh, [0, 1024])
    big = R.tri_workspace_bytes(sh, np.arange(9) * 32768)
    assert 0 < small < big


def test_long_units_leave_the_fused_path():
    """Units of more than 384 fused chunks take the generic path, whose
    workspace holds the raw per-head scores; one chunk fewer stays fused and
    needs no such spill.  The chunk size (a multiple of 64 keys, at most
    1024) depends on the group and head size, so the step is searched for:
    exactly one candidate chunk size shows it."""
    sh = R.make_shape(128, 16, 1, 1)
    G = 16
    jumps = []
    for ch in range(64, 2049, 64):
        fused_n = ch * 384
        w_fused = R.tri_workspace_bytes(sh, [0, fused_n])
        w_long = R.tri_workspace_bytes(sh, [0, fused_n + 1])
        if w_long >= (fused_n + 1) * G * 4 and w_long - w_fused >= (fused_n + 1) * G * 2:
            jumps.append(ch)
    assert len(jumps) == 1, jumps


DEFAULT_OFFSETS = [2.0 ** j for j in range(17)]


def _score_off(shape, cu, cp, offsets=DEFAULT_OFFSETS, reduce="mean", **kw):
    args = dict(k=_Fake(), k_pos=None, q_centre=_Fake(), q_absmean=_Fake(), q_R=_Fake(),
                scores=_Fake(), workspace=None, workspace_bytes=0)
    args.update(kw)
    return R.tri_score_offsets(shape, cu, cp, args["k"], args["k_pos"], args["q_centre"],
                               args["q_absmean"], args["q_R"], offsets, reduce, args["scores"],
                               workspace=args["workspace"],
                               workspace_bytes=args["workspace_bytes"], stream=0)


def test_score_offsets_argument_checks():
    sh = R.make_shape(128, 8, 2, 2)
    cu, cp = [0, 100, 250], [1, 2]
    for red in ("mean", "max"):
        need = R.tri_workspace_bytes_offsets(sh, cu, 17, red)
        assert need > 0
        assert _status(_score_off, sh, cu, cp, reduce=red) == ST["WORKSPACE"]
        assert _status(_score_off, sh, cu, cp, reduce=red, workspace=_Fake(),
                       workspace_bytes=need - 1) == ST["WORKSPACE"]
        assert _status(_score_off, sh, cu, cp, offsets=None, reduce=red) == ST["INVALID"]
        assert _status(_score_off, sh, cu, cp, offsets=[], reduce=red) == ST["INVALID"]
        assert _status(_score_off, sh, cu, cp, offsets=[1.0, float("nan")],
                       reduce=red) == ST["INVALID"]
        assert _status(_score_off, sh, cu, cp, offsets=[1.0, float("inf")],
                       reduce=red) == ST["INVALID"]
        assert _status(_score_off, sh, cu, cp, offsets=np.ones(4097),
                       reduce=red) == ST["INVALID"]
        assert R.tri_workspace_bytes_offsets(sh, cu, 0, red) == 0
        assert R.tri_workspace_bytes_offsets(sh, cu, 4097, red) == 0
        # an empty batch queues nothing and succeeds
        assert _status(_score_off, sh, [0, 0, 0], cp, reduce=red) == 0
    # an unknown reduction code is rejected by the library itself
    lib = R._binding._lib
    st = lib.tri_score_offsets(ctypes.byref(sh), 2, np.array(cu, np.int64).ctypes.data,
                               np.array(cp, np.int32).ctypes.data, FAKE, None, FAKE, FAKE, FAKE,
                               np.array(DEFAULT_OFFSETS).ctypes.data, 17, 7, FAKE, None, None,
                               None, 0, None)
    assert st == ST["INVALID"] and "reduce" in R.last_error()
    assert lib.tri_workspace_bytes_offsets(ctypes.byref(sh), 2,
                                           np.array(cu, np.int64).ctypes.data, 17, 7) == 0


def test_max_over_offsets_shape_limits():
    cu, cp = [0, 64], [64]
    # head_dim must be a multiple of 32 for the MFMA rows
    sh = R.make_shape(72, 4, 2, 1)
    assert _status(_score_off, sh, cu, cp, reduce="max") == ST["UNSUPPORTED"]
    assert R.tri_workspace_bytes_offsets(sh, cu, 17, "max") == 0
    assert R.tri_workspace_bytes_offsets(sh, cu, 17, "mean") > 0
    # one head's rows (two bf16 terms per coefficient) must fit the LDS
    # budget beside the norm operands: 608 offsets at d = 64, 288 at d = 128,
    # 128 at d = 256
    sh = R.make_shape(128, 8, 2, 1)
    assert R.tri_workspace_bytes_offsets(sh, cu, 288, "max") > 0
    assert R.tri_workspace_bytes_offsets(sh, cu, 289, "max") == 0
    assert _status(_score_off, sh, cu, cp, offsets=np.arange(1.0, 290.0),
                   reduce="max") == ST["UNSUPPORTED"]
    sh = R.make_shape(256, 8, 2, 1)
    assert R.tri_workspace_bytes_offsets(sh, cu, 128, "max") > 0
    assert R.tri_workspace_bytes_offsets(sh, cu, 129, "max") == 0
    sh = R.make_shape(64, 8, 2, 1)
    assert R.tri_workspace_bytes_offsets(sh, cu, 608, "max") > 0
    assert R.tri_workspace_bytes_offsets(sh, cu, 609, "max") == 0


def test_offset_workspaces():
    """The mean over any set needs the tri_score layout plus room for the
    offsets; the max adds the per-offset operand rows and the raw spill."""
    sh = R.make_shape(128, 7, 1, 4)
    cu = [0, 32768, 40000]
    base = R.tri_workspace_bytes(sh, cu)
    mean = R.tri_workspace_bytes_offsets(sh, cu, 17, "mean")
    mx = R.tri_workspace_bytes_offsets(sh, cu, 17, "max")
    rows = 4 * cu[-1]
    assert base < mean <= base + 17 * 8 + 256
    assert mx >= rows * 7 * 4 > base
    assert R.tri_workspace_bytes_offsets(sh, cu, 64, "max") > mx



def test_decode_argument_checks():
    """Every failing create is rejected before any device allocation."""
    lib = R._binding._lib
    sh = R.make_shape(128, 8, 2, 2)
    h = ctypes.c_void_p()

    def create(budget=64, interval=16, sink=0, recent=0, n=2, stats=FAKE, shape=sh):
        cfg = R._binding.TriDecodeConfig(budget, interval, sink, recent)
        return lib.tri_decode_create(ctypes.byref(shape) if shape is not None else None, n,
                                     ctypes.byref(cfg), stats, stats, stats, ctypes.byref(h))

    assert create(budget=0) == ST["INVALID"]
    assert create(interval=0) == ST["INVALID"]
    assert create(sink=-1) == ST["INVALID"]
    assert create(sink=40, recent=25) == ST["INVALID"]
    assert "protect" in R.last_error()
    assert create(n=0) == ST["INVALID"]
    assert create(stats=None) == ST["INVALID"]
    assert create(shape=R.make_shape(127, 8, 2, 2)) == ST["INVALID"]
    assert create(budget=2 ** 30, interval=2 ** 30) == ST["UNSUPPORTED"]
    assert h.value is None
    assert lib.tri_decode_create(ctypes.byref(sh), 2, None, FAKE, FAKE, FAKE,
                                 ctypes.byref(h)) == ST["INVALID"]
    # calls on a NULL driver
    assert lib.tri_decode_append(None, FAKE, FAKE, np.zeros(2, np.int32).ctypes.data,
                                 None) == ST["INVALID"]
    assert lib.tri_decode_prefill(None, np.zeros(3, np.int64).ctypes.data,
                                  np.zeros(2, np.int32).ctypes.data, FAKE, FAKE, FAKE,
                                  None) == ST["INVALID"]
    assert lib.tri_decode_get_view(None, None) == ST["INVALID"]
    assert lib.tri_decode_destroy(None) == ST["OK"]



def test_trig_correlation_argument_checks():
    sh = R.make_shape(128, 8, 2, 2)
    need = R.tri_trig_correlation_workspace_bytes(sh, 100)
    assert need == 2 * 8 * 7 * 5 * 8          # L * Hq * ceil(100/16) tiles * 5 sums
    assert R.tri_trig_correlation_workspace_bytes(sh, 0) == 0

    def call(shape=sh, q=_Fake(), qp=_Fake(), nq=100, k=_Fake(), nk=50, c=_Fake(), r=_Fake(),
             ws=None, wsb=0):
        return R.tri_trig_correlation(shape, q, qp, nq, k, None, nk, c, r, workspace=ws,
                                      workspace_bytes=wsb, stream=0)

    assert _status(call, shape=R.make_shape(48, 8, 2, 2)) == ST["UNSUPPORTED"]
    assert _status(call, nq=0) == ST["INVALID"]
    assert _status(call, nk=0) == ST["INVALID"]
    assert _status(call, q=None) == ST["INVALID"]
    assert _status(call, r=None) == ST["INVALID"]
    assert _status(call, k=_Fake(FAKE + 4)) == ST["INVALID"]
    assert _status(call) == ST["WORKSPACE"]
    assert _status(call, ws=_Fake(), wsb=need - 1) == ST["WORKSPACE"]



def test_pyramid_budgets_match_oracle():
    """Host arithmetic, no device: the library's pyramid equals the oracle's."""
    import oracle as O
    for L, mean, ratio in [(28, 2048, 3.0), (32, 1000, 1.0), (1, 77.5, 4.0), (3, 10, 3.0),
                           (7, 513.3, 0.5), (40, 4096, 8.0)]:
        np.testing.assert_array_equal(R.tri_pyramid_budgets(L, mean, ratio),
                                      O.pyramid_budgets(L, mean, ratio))
    for bad in [(0, 10, 2.0), (4, -1, 2.0), (4, 10, 0.0), (4, float("nan"), 2.0)]:
        assert _status(R.tri_pyramid_budgets, *bad) == ST["INVALID"]


def test_select_compact_layers_argument_checks():
    sh = R.make_shape(64, 4, 2, 3)
    cu = [0, 50, 80]
    bud = [[10, 20, 30], [5, 5, 5]]
    need = R.tri_workspace_bytes_layers(sh, cu)
    assert need == 512                 # control words, then 6 plan entries of 40 bytes

    def sel(budget=bud, **kw):
        args = dict(scores=_Fake(), k=_Fake(), v=_Fake(), k_pos=_Fake(), kept=_Fake(),
                    k_out=_Fake(FAKE * 2), v_out=_Fake(FAKE * 3), pos_out=_Fake(FAKE * 4),
                    workspace=None, workspace_bytes=0)
        args.update(kw)
        return R.tri_select_compact_layers(sh, cu, budget, args["scores"], args["k"], args["v"],
                                           args["k_pos"], args["kept"], args["k_out"],
                                           args["v_out"], args["pos_out"],
                                           workspace=args["workspace"],
                                           workspace_bytes=args["workspace_bytes"], stream=0)

    assert _status(sel, budget=[[10, -1, 3], [5, 5, 5]]) == ST["INVALID"]
    assert _status(sel, v_out=None) == ST["INVALID"]
    assert _status(sel) == ST["WORKSPACE"]
    assert _status(sel, budget=[[0, 0, 0], [0, 0, 0]]) == 0


def test_shape_struct_layout_and_rope_layout_field():
    """tri_shape: four int32, the double at byte 16, rope_layout at byte 24
    (32 bytes with padding), matching the C declaration."""
    import ctypes
    assert ctypes.sizeof(R.TriShape) == 32
    assert R.TriShape.rope_theta.offset == 16 and R.TriShape.rope_layout.offset == 24
    assert R.make_shape(64, 4, 2, 1).rope_layout == R.TRI_ROPE_INTERLEAVED
    assert R.make_shape(64, 4, 2, 1, rope_layout="half").rope_layout == R.TRI_ROPE_HALF_SPLIT
    bad = R.make_shape(64, 4, 2, 1, rope_layout=2)
    assert _status(_score, bad, [0, 8], [8]) == ST["INVALID"]
    assert "rope_layout" in R.last_error()
    assert R.tri_workspace_bytes(bad, [0, 8]) == 0
    # half split: every head_dim the interleaved layout takes is accepted
    for d in (8, 24, 96, 128, 256):
        sh = R.make_shape(d, 4, 2, 1, rope_layout="half")
        assert R.tri_workspace_bytes(sh, [0, 8]) > 0
        assert _status(_score, sh, [0, 8], [8]) == ST["WORKSPACE"]


def test_max_offsets_half_split_needs_d_multiple_of_64():
    offs = np.array([1.0, 2.0, 4.0])
    for d, ok in ((96, False), (160, False), (64, True), (128, True)):
        sh = R.make_shape(d, 4, 2, 1, rope_layout="half")
        got = R.tri_workspace_bytes_offsets(sh, [0, 8], len(offs), "max")
        assert (got > 0) == ok, (d, got)
        if not ok:
            assert "half-split" in R.last_error()
        # the mean over the same set has no such limit
        assert R.tri_workspace_bytes_offsets(sh, [0, 8], len(offs), "mean") > 0



def _pages(**kw):
    a = dict(page_table=_Fake(FAKE * 5), page_size=16, num_pages=10, page_stride=64,
             token_stride=4, head_stride=1, layer_stride=640)
    a.update(kw)
    pt = a.pop("page_table")
    p = R.TriKvPages(ctypes.c_void_p(pt.data_ptr()) if pt is not None else None, 4,
                     a["num_pages"], a["page_size"], a["page_stride"], a["token_stride"],
                     a["head_stride"], a["layer_stride"])
    return p


def test_kv_pages_struct_layout():
    """tri_kv_pages: pointer, three int32, then four int64 from byte 24."""
    assert ctypes.sizeof(R.TriKvPages) == 56
    assert R.TriKvPages.page_stride.offset == 24 and R.TriKvPages.layer_stride.offset == 48


def test_score_paged_argument_checks():
    sh = R.make_shape(128, 8, 4, 2)
    cu, cp = [0, 40, 64], [40, 24]

    def call(pages, **kw):
        a = dict(k=_Fake(), qc=_Fake(), qa=_Fake(), qr=_Fake(), scores=_Fake(), workspace=None,
                 workspace_bytes=0)
        a.update(kw)
        return R.tri_score_paged(sh, cu, cp, pages, a["k"], a["qc"], a["qa"], a["qr"], a["scores"],
                                 workspace=a["workspace"], workspace_bytes=a["workspace_bytes"],
                                 stream=0)

    assert _status(call, None) == ST["INVALID"]
    assert _status(call, _pages(page_table=None)) == ST["INVALID"]
    for bad in (dict(page_size=0), dict(page_size=24), dict(page_size=1 << 17),
                dict(num_pages=0), dict(token_stride=-1)):
        assert _status(call, _pages(**bad)) == ST["INVALID"], bad
    assert "page" in R.last_error()
    # 40 keys in pages of 8 need 5 pages; the table holds 4 per sequence
    assert _status(call, _pages(page_size=8)) == ST["INVALID"]
    assert "pages" in R.last_error()
    assert _status(call, _pages(layer_stride=1 << 60)) == ST["UNSUPPORTED"]
    assert _status(call, _pages()) == ST["WORKSPACE"]
    assert _status(call, _pages(), k=_Fake(FAKE + 8)) == ST["INVALID"]     # misaligned pool


def test_select_compact_paged_argument_checks():
    sh = R.make_shape(64, 4, 2, 1)
    cu = [0, 50, 80]

    def call(budget=(10, 10), in_pages=_pages(), out_pages=_pages(), rows=True, **kw):
        p = FAKE * 2 if rows else None
        a = dict(k=_Fake(p) if rows else None, v=_Fake(p) if rows else None,
                 pos=_Fake(p) if rows else None, ko=_Fake(p) if rows else None,
                 vo=_Fake(p) if rows else None, po=_Fake(p) if rows else None)
        a.update(kw)
        return R.tri_select_compact_paged(sh, cu, list(budget), _Fake(), in_pages, a["k"], a["v"],
                                          a["pos"], _Fake(), out_pages, a["ko"], a["vo"], a["po"],
                                          workspace=None, workspace_bytes=0, stream=0)

    assert _status(call, vo=None) == ST["INVALID"]                    # unpaired pools
    assert _status(call, out_pages=None) == ST["INVALID"]
    assert _status(call, budget=(10, -1)) == ST["INVALID"]
    # 50 kept keys in output pages of 8 need 7 pages; the table holds 4
    assert _status(call, budget=(50, 10), out_pages=_pages(page_size=8)) == ST["INVALID"]
    assert _status(call) == ST["WORKSPACE"]
    assert _status(call, budget=(0, 0)) == 0                          # nothing kept
    # indices only: no pools and no page descriptors needed
    assert _status(call, rows=False, in_pages=None, out_pages=None) == ST["WORKSPACE"]



def test_workspace_bytes_paged():
    """Pages of >= 16 tokens take the fused path (its workspace); smaller
    pages the VALU path, which also holds raw scores in the workspace."""
    sh = R.make_shape(128, 8, 2, 2)
    cu = [0, 3000, 5000]
    fused = R.tri_workspace_bytes(sh, cu)
    assert R.tri_workspace_bytes_paged(sh, cu, 16) == fused
    assert R.tri_workspace_bytes_paged(sh, cu, 256) == fused
    small = R.tri_workspace_bytes_paged(sh, cu, 8)
    assert small >= fused + 2 * 2 * 5000 * 4 * 4           # raw scores: rows x G floats
    assert R.tri_workspace_bytes_paged(sh, cu, 16, 3, "max") == \
        R.tri_workspace_bytes_offsets(sh, cu, 3, "max")
    assert R.tri_workspace_bytes_paged(sh, cu, 12) == 0
    assert R.tri_workspace_bytes_paged(sh, cu, 16, 5000) == 0


def test_sequence_count_limit():
    """One call plans at most 8192 sequences (the plan travels through a
    fixed pinned staging slot); 8193 is refused before any device work."""
    sh = R.make_shape(64, 4, 2, 1)
    ok_cu = np.arange(8193, dtype=np.int64)          # 8192 sequences of one key
    bad_cu = np.arange(8194, dtype=np.int64)
    assert R.tri_workspace_bytes(sh, ok_cu) > 0
    assert R.tri_workspace_bytes(sh, bad_cu) == 0
    assert _status(_score, sh, bad_cu, np.full(8193, 5, np.int32)) == ST["UNSUPPORTED"]
    assert "8192" in R.last_error()
    assert _status(_sel, sh, bad_cu, np.ones(8193, np.int32)) == ST["UNSUPPORTED"]


def test_stream_probe_rejects_bad_arguments():
    sink = _Fake(FAKE + 64)
    with pytest.raises(R.TriError, match="INVALID"):
        R.tri_stream_probe(_Fake(FAKE + 4), sink, nbytes=64, stream=0)   # misaligned
    with pytest.raises(R.TriError, match="INVALID"):
        R.tri_stream_probe(_Fake(), sink, nbytes=40, stream=0)   # not a multiple of 16
    with pytest.raises(R.TriError, match="INVALID"):
        R.tri_stream_probe(_Fake(0), sink, nbytes=64, stream=0)   # NULL src
    R.tri_stream_probe(_Fake(0), _Fake(0), nbytes=0, stream=0)   # empty: a no-op


def test_noalloc_rejects_calls_past_its_scratch():
    """tri_score_noalloc holds 64 MiB of device scratch: a call needing more
    (4096 units: 64 MiB of packed operands alone) fails with
    TRI_ERR_WORKSPACE before queueing anything; one that fits gets past that
    check (and fails here only on the fake K pointer's alignment)."""
    big = R.make_shape(128, 64, 64, 64)
    cu, cp = np.array([0, 16], np.int64), np.array([16], np.int32)
    assert R.tri_workspace_bytes(big, cu) > 64 << 20
    a = (_Fake(), None, _Fake(), _Fake(), _Fake(), _Fake())
    assert _status(R.tri_score_noalloc, big, cu, cp, *a, stream=0) == ST["WORKSPACE"]
    assert "tri_score_noalloc holds 67108864" in R.last_error()
    small = R.make_shape(128, 7, 1, 1)
    a = (_Fake(FAKE + 4), None, _Fake(), _Fake(), _Fake(), _Fake())
    assert _status(R.tri_score_noalloc, small, cu, cp, *a, stream=0) == ST["INVALID"]


def test_fused_routing_follows_resident_work_groups():
    """The planner keeps a unit on the fused path only while its chunks
    number at most the work-groups the device holds at once.  With 96
    resident (a 32-CU partition, three per CU) a unit of 97 chunks moves to
    the generic path, whose workspace spills the raw scores; 96 chunks stay
    fused.  The device's own count (three per CU on 256 CUs, or no device
    here) leaves both fused."""
    sh = R.make_shape(128, 7, 1, 1)
    G = 7
    ch = None
    for c in range(64, 2049, 64):   # the fused chunk size: where 384 chunks stop fitting
        if R.tri_workspace_bytes(sh, [0, c * 384 + 1]) >= (c * 384 + 1) * G * 4:
            if R.tri_workspace_bytes(sh, [0, c * 384]) < c * 384 * G * 4:
                ch = c
    assert ch is not None
    n96, n97 = 96 * ch, 96 * ch + 1
    base96, base97 = R.tri_workspace_bytes(sh, [0, n96]), R.tri_workspace_bytes(sh, [0, n97])
    assert base97 < n97 * G * 4                      # fused at the device's count
    prev = R.tri_debug_set_resident_groups(96)
    try:
        assert R.tri_workspace_bytes(sh, [0, n96]) == base96
        assert R.tri_workspace_bytes(sh, [0, n97]) >= n97 * G * 4   # generic: raw spill
    finally:
        R.tri_debug_set_resident_groups(prev)
    assert prev == 0
    assert R.tri_workspace_bytes(sh, [0, n97]) == base97
