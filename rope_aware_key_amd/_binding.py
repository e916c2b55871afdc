"""ctypes binding of libtriattn.so: argument marshalling only.

Every call forwards device pointers (torch tensors' data_ptr), host arrays
and the current HIP stream to the C ABI in include/triattn.h.  Nothing here
computes any part of the path; if the library is missing, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# One HIP runtime per process: torch ships its own libamdhip64 with the same
# soname as the system one this library links.  Loading torch first makes the
# library bind to torch's runtime instead of pulling in a second copy, which
# would leave the two runtimes fighting over the device.
import torch  # noqa: F401,E402

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtriattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")

_lib = ctypes.CDLL(LIB_PATH)

TRI_OK = 0
STATUS = {0: "TRI_OK", 1: "TRI_ERR_INVALID_ARGUMENT", 2: "TRI_ERR_UNSUPPORTED",
          3: "TRI_ERR_WORKSPACE", 4: "TRI_ERR_HIP"}


class TriShape(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("rope_layout", ctypes.c_int32)]


_P = ctypes.c_void_p
_lib.tri_calibrate_workspace_bytes.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int64]
_lib.tri_calibrate_workspace_bytes.restype = ctypes.c_size_t
_lib.tri_calibrate.argtypes = [ctypes.POINTER(TriShape), _P, _P, ctypes.c_int64, _P, _P, _P, _P,
                               ctypes.c_size_t, _P]
_lib.tri_calibrate.restype = ctypes.c_int
_lib.tri_workspace_bytes.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P]
_lib.tri_workspace_bytes.restype = ctypes.c_size_t
_lib.tri_score.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                           _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.tri_score.restype = ctypes.c_int
_lib.tri_score_noalloc.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                  _P, _P, _P, _P]
_lib.tri_score_noalloc.restype = ctypes.c_int
_lib.tri_workspace_bytes_offsets.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P,
                                             ctypes.c_int32, ctypes.c_int32]
_lib.tri_workspace_bytes_offsets.restype = ctypes.c_size_t
_lib.tri_score_offsets.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P, _P, _P, _P, _P,
                                   _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P]
_lib.tri_score_offsets.restype = ctypes.c_int
_lib.tri_select_compact.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P, _P, _P, _P, _P,
                                    _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.tri_select_compact.restype = ctypes.c_int
_lib.tri_status_string.argtypes = [ctypes.c_int]
_lib.tri_status_string.restype = ctypes.c_char_p
_lib.tri_last_error.argtypes = []
_lib.tri_last_error.restype = ctypes.c_char_p
_lib.tri_debug_set_wait_limit.argtypes = [ctypes.c_uint32]
_lib.tri_debug_set_wait_limit.restype = ctypes.c_uint32
_lib.tri_debug_set_phase_buffer.argtypes = [_P]
_lib.tri_debug_set_phase_buffer.restype = _P
_lib.tri_debug_set_resident_groups.argtypes = [ctypes.c_int32]
_lib.tri_debug_set_resident_groups.restype = ctypes.c_int32
_lib.tri_score_status.argtypes = [_P, ctypes.POINTER(ctypes.c_uint32), _P]
_lib.tri_score_status.restype = ctypes.c_int

class TriDecodeConfig(ctypes.Structure):
    _fields_ = [("budget", ctypes.c_int32), ("interval", ctypes.c_int32),
                ("protect_sink", ctypes.c_int32), ("protect_recent", ctypes.c_int32)]


class TriDecodeView(ctypes.Structure):
    _fields_ = [("unit_stride", ctypes.c_int64), ("k", ctypes.POINTER(ctypes.c_void_p)),
                ("v", ctypes.POINTER(ctypes.c_void_p)), ("pos", ctypes.POINTER(ctypes.c_void_p)),
                ("len", ctypes.POINTER(ctypes.c_int32)),
                ("scores", ctypes.POINTER(ctypes.c_void_p)),
                ("scores_stride", ctypes.POINTER(ctypes.c_int64)), ("prunes", ctypes.c_int64)]


_lib.tri_decode_create.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32,
                                   ctypes.POINTER(TriDecodeConfig), _P, _P, _P,
                                   ctypes.POINTER(ctypes.c_void_p)]
_lib.tri_decode_create.restype = ctypes.c_int
_lib.tri_decode_prefill.argtypes = [_P, _P, _P, _P, _P, _P, _P]
_lib.tri_decode_prefill.restype = ctypes.c_int
_lib.tri_decode_append.argtypes = [_P, _P, _P, _P, _P]
_lib.tri_decode_append.restype = ctypes.c_int
_lib.tri_decode_get_view.argtypes = [_P, ctypes.POINTER(TriDecodeView)]
_lib.tri_decode_get_view.restype = ctypes.c_int
_lib.tri_decode_destroy.argtypes = [_P]
_lib.tri_decode_destroy.restype = ctypes.c_int

_lib.tri_trig_correlation_workspace_bytes.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int64]
_lib.tri_trig_correlation_workspace_bytes.restype = ctypes.c_size_t
_lib.tri_trig_correlation.argtypes = [ctypes.POINTER(TriShape), _P, _P, ctypes.c_int64, _P, _P,
                                      ctypes.c_int64, _P, _P, _P, ctypes.c_size_t, _P]
_lib.tri_trig_correlation.restype = ctypes.c_int

_lib.tri_stream_probe.argtypes = [_P, ctypes.c_size_t, _P, _P]
_lib.tri_stream_probe.restype = ctypes.c_int
_lib.tri_pyramid_budgets.argtypes = [ctypes.c_int32, ctypes.c_double, ctypes.c_double, _P]
_lib.tri_pyramid_budgets.restype = ctypes.c_int
_lib.tri_workspace_bytes_layers.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P]
_lib.tri_workspace_bytes_layers.restype = ctypes.c_size_t
_lib.tri_select_compact_layers.argtypes = _lib.tri_select_compact.argtypes
_lib.tri_select_compact_layers.restype = ctypes.c_int


class TriKvPages(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("page_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("layer_stride", ctypes.c_int64)]


_PG = ctypes.POINTER(TriKvPages)
_lib.tri_score_paged.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P, _P, _PG, _P, _P, _P,
                                 _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P,
                                 ctypes.c_size_t, _P]
_lib.tri_score_paged.restype = ctypes.c_int
_lib.tri_select_compact_paged.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P, _P, _P, _PG,
                                          _P, _P, _P, _P, _PG, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.tri_select_compact_paged.restype = ctypes.c_int
_lib.tri_workspace_bytes_paged.argtypes = [ctypes.POINTER(TriShape), ctypes.c_int32, _P,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
_lib.tri_workspace_bytes_paged.restype = ctypes.c_size_t

EXPORTS = ("tri_calibrate", "tri_calibrate_workspace_bytes", "tri_workspace_bytes", "tri_score", "tri_select_compact",
           "tri_status_string", "tri_last_error", "tri_workspace_bytes_offsets",
           "tri_score_offsets", "tri_decode_create", "tri_decode_prefill", "tri_decode_append",
           "tri_decode_get_view", "tri_decode_destroy", "tri_trig_correlation_workspace_bytes",
           "tri_trig_correlation", "tri_stream_probe", "tri_score_noalloc", "tri_score_status",
           "tri_debug_set_resident_groups", "tri_pyramid_budgets", "tri_workspace_bytes_layers",
           "tri_select_compact_layers", "tri_score_paged", "tri_select_compact_paged",
           "tri_workspace_bytes_paged", "tri_debug_set_wait_limit", "tri_debug_set_phase_buffer")

TRI_REDUCE_MEAN = 0
TRI_REDUCE_MAX = 1
REDUCE = {"mean": TRI_REDUCE_MEAN, "max": TRI_REDUCE_MAX}


class TriError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.tri_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def _check(st, where):
    if st != TRI_OK:
        raise TriError(st, where)


TRI_ROPE_INTERLEAVED = 0
TRI_ROPE_HALF_SPLIT = 1
ROPE_LAYOUT = {"interleaved": TRI_ROPE_INTERLEAVED, "half": TRI_ROPE_HALF_SPLIT}


def make_shape(head_dim, num_q_heads, num_kv_heads, num_layers, rope_theta=10000.0,
               rope_layout="interleaved") -> TriShape:
    """rope_layout: "interleaved" (band f = x[2f], x[2f+1]), "half"
    (x[f], x[f + d/2]) or the TRI_ROPE_* value."""
    lay = ROPE_LAYOUT[rope_layout] if isinstance(rope_layout, str) else int(rope_layout)
    return TriShape(head_dim, num_q_heads, num_kv_heads, num_layers, float(rope_theta), lay)


def _ptr(t):
    """Device (or host) address of a tensor, or NULL for None."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _host(a, dtype):
    """Contiguous host numpy array (kept alive by the caller's reference)."""
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=dtype))
    return arr, ctypes.c_void_p(arr.ctypes.data)


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream))


def status_string(st: int) -> str:
    return _lib.tri_status_string(st).decode()


def last_error() -> str:
    return _lib.tri_last_error().decode()


def tri_calibrate_workspace_bytes(shape: TriShape, n_samples) -> int:
    return int(_lib.tri_calibrate_workspace_bytes(ctypes.byref(shape), int(n_samples)))


def tri_calibrate(shape: TriShape, q, q_pos, n_samples, q_centre, q_absmean, q_R, workspace=None,
                  workspace_bytes=None, stream=None):
    """workspace: device tensor of tri_calibrate_workspace_bytes(); when None
    one is allocated through torch on q's device."""
    if workspace is None and workspace_bytes is None and hasattr(q, "device"):
        import torch
        need = tri_calibrate_workspace_bytes(shape, n_samples)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wsb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = _lib.tri_calibrate(ctypes.byref(shape), _ptr(q), _ptr(q_pos), int(n_samples),
                            _ptr(q_centre), _ptr(q_absmean), _ptr(q_R), _ptr(workspace), int(wsb),
                            _stream(stream))
    _check(st, "tri_calibrate")


def tri_workspace_bytes(shape: TriShape, cu_len) -> int:
    arr, p = _host(cu_len, np.int64)
    return int(_lib.tri_workspace_bytes(ctypes.byref(shape), len(arr) - 1, p))


def tri_score(shape: TriShape, cu_len, cur_pos, k, k_pos, q_centre, q_absmean, q_R, scores,
              raw_scores=None, head_stats=None, workspace=None, workspace_bytes=None, stream=None):
    cu, pcu = _host(cu_len, np.int64)
    cp, pcp = _host(cur_pos, np.int32)
    wsb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = _lib.tri_score(ctypes.byref(shape), len(cu) - 1, pcu, pcp, _ptr(k), _ptr(k_pos),
                        _ptr(q_centre), _ptr(q_absmean), _ptr(q_R), _ptr(scores),
                        _ptr(raw_scores), _ptr(head_stats), _ptr(workspace), int(wsb),
                        _stream(stream))
    _check(st, "tri_score")


def tri_score_noalloc(shape: TriShape, cu_len, cur_pos, k, k_pos, q_centre, q_absmean, q_R,
                      scores, raw_scores=None, head_stats=None, stream=None):
    """tri_score without a workspace (the library's device scratch; see
    include/triattn.h for its limit and sharing rules)."""
    cu, pcu = _host(cu_len, np.int64)
    cp, pcp = _host(cur_pos, np.int32)
    st = _lib.tri_score_noalloc(ctypes.byref(shape), len(cu) - 1, pcu, pcp, _ptr(k), _ptr(k_pos),
                                _ptr(q_centre), _ptr(q_absmean), _ptr(q_R), _ptr(scores),
                                _ptr(raw_scores), _ptr(head_stats), _stream(stream))
    _check(st, "tri_score_noalloc")


def tri_workspace_bytes_offsets(shape: TriShape, cu_len, n_offsets, reduce="mean") -> int:
    arr, p = _host(cu_len, np.int64)
    return int(_lib.tri_workspace_bytes_offsets(ctypes.byref(shape), len(arr) - 1, p,
                                                int(n_offsets), REDUCE[reduce]))


def tri_score_offsets(shape: TriShape, cu_len, cur_pos, k, k_pos, q_centre, q_absmean, q_R,
                      offsets, reduce, scores, raw_scores=None, head_stats=None, workspace=None,
                      workspace_bytes=None, stream=None):
    """tri_score over a caller-given offset set; reduce is "mean" or "max"."""
    cu, pcu = _host(cu_len, np.int64)
    cp, pcp = _host(cur_pos, np.int32)
    off, poff = _host(offsets, np.float64)
    wsb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = _lib.tri_score_offsets(ctypes.byref(shape), len(cu) - 1, pcu, pcp, _ptr(k), _ptr(k_pos),
                                _ptr(q_centre), _ptr(q_absmean), _ptr(q_R), poff,
                                0 if off is None else len(off), REDUCE[reduce], _ptr(scores),
                                _ptr(raw_scores), _ptr(head_stats), _ptr(workspace), int(wsb),
                                _stream(stream))
    _check(st, "tri_score_offsets")


def tri_trig_correlation_workspace_bytes(shape: TriShape, n_q) -> int:
    return int(_lib.tri_trig_correlation_workspace_bytes(ctypes.byref(shape), int(n_q)))


def tri_trig_correlation(shape: TriShape, q, q_pos, n_q, k, k_pos, n_k, q_centre, r,
                         workspace=None, workspace_bytes=None, stream=None):
    """Per-(layer, query head) Pearson r of the trig reconstruction against
    the direct logits (include/triattn.h)."""
    wsb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = _lib.tri_trig_correlation(ctypes.byref(shape), _ptr(q), _ptr(q_pos), int(n_q), _ptr(k),
                                   _ptr(k_pos), int(n_k), _ptr(q_centre), _ptr(r), _ptr(workspace),
                                   int(wsb), _stream(stream))
    _check(st, "tri_trig_correlation")


def tri_stream_probe(src, sink, nbytes=None, stream=None):
    """Read-bandwidth probe: reads src (device, 16-byte aligned) once and
    XORs its 32-bit words into sink (one device uint32/int32, not cleared)."""
    n = nbytes if nbytes is not None else src.numel() * src.element_size()
    st = _lib.tri_stream_probe(_ptr(src), int(n), _ptr(sink), _stream(stream))
    _check(st, "tri_stream_probe")


TRI_SCORE_WAIT_GAVE_UP = 1


def tri_score_status(workspace=None, stream=None) -> int:
    """Flags of the last score call on `workspace` (None: tri_score_noalloc's
    scratch): TRI_SCORE_WAIT_GAVE_UP if it gave up a bounded wait.  Waits for
    the stream's queued work."""
    flags = ctypes.c_uint32(0)
    st = _lib.tri_score_status(_ptr(workspace), ctypes.byref(flags), _stream(stream))
    _check(st, "tri_score_status")
    return int(flags.value)


def tri_debug_set_resident_groups(groups: int) -> int:
    """Test hook: the planner's resident work-group count (0 = query the device)."""
    return int(_lib.tri_debug_set_resident_groups(int(groups)))


def tri_select_compact(shape: TriShape, cu_len, budget, scores, k, v, k_pos, kept_idx, k_out,
                       v_out, pos_out, workspace=None, workspace_bytes=None, stream=None):
    cu, pcu = _host(cu_len, np.int64)
    bu, pbu = _host(budget, np.int32)
    wsb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = _lib.tri_select_compact(ctypes.byref(shape), len(cu) - 1, pcu, pbu, _ptr(scores), _ptr(k),
                                 _ptr(v), _ptr(k_pos), _ptr(kept_idx), _ptr(k_out), _ptr(v_out),
                                 _ptr(pos_out), _ptr(workspace), int(wsb), _stream(stream))
    _check(st, "tri_select_compact")


class Decode:
    """The decode-loop driver (tri_decode_* in include/triattn.h)."""

    def __init__(self, shape: TriShape, num_seqs, budget, interval, q_centre, q_absmean, q_R,
                 protect_sink=0, protect_recent=0):
        self.num_seqs = int(num_seqs)
        cfg = TriDecodeConfig(int(budget), int(interval), int(protect_sink), int(protect_recent))
        h = ctypes.c_void_p()
        _check(_lib.tri_decode_create(ctypes.byref(shape), self.num_seqs, ctypes.byref(cfg),
                                      _ptr(q_centre), _ptr(q_absmean), _ptr(q_R),
                                      ctypes.byref(h)), "tri_decode_create")
        self._h = h

    def prefill(self, cu_len, cur_pos, k, v, k_pos, stream=None):
        self._cu, pcu = _host(cu_len, np.int64)
        self._cp, pcp = _host(cur_pos, np.int32)
        _check(_lib.tri_decode_prefill(self._h, pcu, pcp, _ptr(k), _ptr(v), _ptr(k_pos),
                                       _stream(stream)), "tri_decode_prefill")

    def append(self, k_new, v_new, pos_new, stream=None):
        self._pn, ppn = _host(pos_new, np.int32)
        _check(_lib.tri_decode_append(self._h, _ptr(k_new), _ptr(v_new), ppn, _stream(stream)),
               "tri_decode_append")

    def view(self) -> dict:
        vw = TriDecodeView()
        _check(_lib.tri_decode_get_view(self._h, ctypes.byref(vw)), "tri_decode_get_view")
        n = self.num_seqs
        return {"unit_stride": int(vw.unit_stride), "k": [vw.k[i] for i in range(n)],
                "v": [vw.v[i] for i in range(n)], "pos": [vw.pos[i] for i in range(n)],
                "len": [int(vw.len[i]) for i in range(n)],
                "scores": [vw.scores[i] for i in range(n)],
                "scores_stride": [int(vw.scores_stride[i]) for i in range(n)],
                "prunes": int(vw.prunes)}

    def close(self):
        if self._h:
            _check(_lib.tri_decode_destroy(self._h), "tri_decode_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tri_debug_set_wait_limit(polls: int) -> int:
    """Test hook: bound on the fused score kernel's wait (see triattn.h)."""
    return int(_lib.tri_debug_set_wait_limit(int(polls)))


PHASE_NAMES = ("stream", "other_waves", "next_ticket", "moments", "stats_wait", "zscore_max",
               "operands_stores")


def tri_debug_set_phase_buffer(buf) -> int:
    """Measurement hook: a device tensor of 8 int64 counters (zeroed by the
    caller) for the fused score kernel's phase cycles, or None to turn it
    off (see triattn.h).  Returns the previous buffer's address (0 if none)."""
    if buf is not None and (buf.device.type != "cuda" or buf.numel() < 8 or buf.element_size() != 8
                            or not buf.is_contiguous()):
        raise ValueError("phase buffer: 8 contiguous 64-bit counters in device memory")
    return int(_lib.tri_debug_set_phase_buffer(None if buf is None else buf.data_ptr()) or 0)


def tri_pyramid_budgets(num_layers, mean_budget, ratio):
    out = np.zeros(int(num_layers), dtype=np.int32)
    _check(_lib.tri_pyramid_budgets(int(num_layers), float(mean_budget), float(ratio),
                                    ctypes.c_void_p(out.ctypes.data)), "tri_pyramid_budgets")
    return out


def tri_workspace_bytes_layers(shape: TriShape, cu_len) -> int:
    arr, p = _host(cu_len, np.int64)
    return int(_lib.tri_workspace_bytes_layers(ctypes.byref(shape), len(arr) - 1, p))


def tri_select_compact_layers(shape: TriShape, cu_len, budget, scores, k, v, k_pos, kept_idx,
                              k_out, v_out, pos_out, workspace=None, workspace_bytes=None,
                              stream=None):
    """tri_select_compact with budget [num_seqs][L] (one per sequence and layer)."""
    cu, pcu = _host(cu_len, np.int64)
    bu, pbu = _host(np.asarray(budget).reshape(-1), np.int32)
    wsb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = _lib.tri_select_compact_layers(ctypes.byref(shape), len(cu) - 1, pcu, pbu, _ptr(scores),
                                        _ptr(k), _ptr(v), _ptr(k_pos), _ptr(kept_idx), _ptr(k_out),
                                        _ptr(v_out), _ptr(pos_out), _ptr(workspace), int(wsb),
                                        _stream(stream))
    _check(st, "tri_select_compact_layers")


def make_pages(page_table, page_size, num_pages, page_stride, token_stride, head_stride,
               layer_stride) -> TriKvPages:
    """tri_kv_pages for a device page table [num_seqs, max_pages] (int32
    tensor, kept alive by the caller); strides in rows."""
    return TriKvPages(ctypes.c_void_p(page_table.data_ptr()), int(page_table.shape[-1]),
                      int(num_pages), int(page_size), int(page_stride), int(token_stride),
                      int(head_stride), int(layer_stride))


def tri_workspace_bytes_paged(shape: TriShape, cu_len, page_size, n_offsets=0,
                              reduce="mean") -> int:
    arr, p = _host(cu_len, np.int64)
    return int(_lib.tri_workspace_bytes_paged(ctypes.byref(shape), len(arr) - 1, p,
                                              int(page_size), int(n_offsets), REDUCE[reduce]))


def _pages(p):
    return None if p is None else ctypes.byref(p)


def tri_score_paged(shape: TriShape, cu_len, cur_pos, pages: TriKvPages, k_pool, q_centre,
                    q_absmean, q_R, scores, offsets=None, reduce="mean", raw_scores=None,
                    head_stats=None, workspace=None, workspace_bytes=None, stream=None):
    """tri_score (offsets None) or tri_score_offsets with keys in a paged pool."""
    cu, pcu = _host(cu_len, np.int64)
    cp, pcp = _host(cur_pos, np.int32)
    off, poff = _host(offsets, np.float64)
    wsb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = _lib.tri_score_paged(ctypes.byref(shape), len(cu) - 1, pcu, pcp, _pages(pages),
                              _ptr(k_pool), _ptr(q_centre), _ptr(q_absmean), _ptr(q_R), poff,
                              0 if off is None else len(off), REDUCE[reduce], _ptr(scores),
                              _ptr(raw_scores), _ptr(head_stats), _ptr(workspace), int(wsb),
                              _stream(stream))
    _check(st, "tri_score_paged")


def tri_select_compact_paged(shape: TriShape, cu_len, budget, scores, in_pages, k_pool, v_pool,
                             pos_pool, kept_idx, out_pages, k_out_pool, v_out_pool, pos_out_pool,
                             workspace=None, workspace_bytes=None, stream=None):
    """tri_select_compact with K, V, positions read from and written to paged pools."""
    cu, pcu = _host(cu_len, np.int64)
    bu, pbu = _host(budget, np.int32)
    wsb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = _lib.tri_select_compact_paged(ctypes.byref(shape), len(cu) - 1, pcu, pbu, _ptr(scores),
                                       _pages(in_pages), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(pos_pool), _ptr(kept_idx), _pages(out_pages),
                                       _ptr(k_out_pool), _ptr(v_out_pool), _ptr(pos_out_pool),
                                       _ptr(workspace), int(wsb), _stream(stream))
    _check(st, "tri_select_compact_paged")

