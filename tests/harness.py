"""Shared helpers for the parity tests: run a synthetic case through the HIP
library (via the binding) and evaluate units with the CPU oracle."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle as O
from checks import check_raw, check_scores, head_stat_errors, score_error, z_floor  # noqa: F401
from synth import Case


_HIP = None


def dev_read(ptr: int, count: int, dtype) -> np.ndarray:
    """Copy `count` elements at a raw device address to a host array (after
    the device is idle), through the HIP runtime torch has loaded."""
    global _HIP
    import ctypes
    import os
    if _HIP is None:
        _HIP = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        _HIP.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _HIP.hipMemcpy.restype = ctypes.c_int
    torch.cuda.synchronize()
    out = np.empty(count, dtype=dtype)
    if count:
        rc = _HIP.hipMemcpy(out.ctypes.data, ptr, out.nbytes, 2)  # device to host
        assert rc == 0, f"hipMemcpy failed: {rc}"
    return out


def layout_of(case: Case) -> str:
    return case.meta.get("rope_layout", "interleaved")


def shape_of(case: Case):
    import rope_aware_key_amd as R
    sh = case.shape
    return R.make_shape(sh.head_dim, sh.num_q_heads, sh.num_kv_heads, sh.num_layers, sh.rope_theta,
                        rope_layout=layout_of(case))


def half_split(case: Case) -> Case:
    """The same case stored in the half-split RoPE layout: the columns of
    every key row and calibration query are permuted from (x0, x1, x2, ..)
    to (x0, x2, .., x1, x3, ..), so band f moves from (2f, 2f+1) to
    (f, f + d/2).  Values are not rotated and stay as they are."""
    import dataclasses
    d = case.shape.head_dim
    perm = torch.as_tensor(np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)]),
                           device=case.k.device)
    cq = None if case.calib_q is None else case.calib_q[..., perm].contiguous()
    return dataclasses.replace(case, k=case.k[:, perm].contiguous(), calib_q=cq,
                               meta=dict(case.meta, rope_layout="half"))


def pinned(a, dtype):
    """Page-locked host copy (the library reads host arrays during the call)."""
    t = torch.as_tensor(np.asarray(a, dtype=dtype))
    return t.pin_memory().numpy()


def gpu_calibrate(case: Case):
    """Fill case.q_centre/q_absmean/q_R from case.calib_q on the GPU."""
    import rope_aware_key_amd as R
    n = case.calib_q.shape[1]
    R.tri_calibrate(shape_of(case), case.calib_q, case.calib_pos, n, case.q_centre, case.q_absmean,
                    case.q_R)
    torch.cuda.synchronize()


def gpu_run(case: Case, raw=True, stats=True, compact=True, scores_in=None):
    """Score + select/compact one case on the GPU.  Returns a dict of tensors."""
    import rope_aware_key_amd as R
    dev = case.k.device
    sh = shape_of(case)
    G = case.shape.group
    rows = case.total_rows()
    out_rows = case.total_out_rows()
    d = case.shape.head_dim
    cu = pinned(case.cu_len, np.int64)
    cp = pinned(case.cur_pos, np.int32)
    bu = pinned(case.budget, np.int32)
    wsb = R.tri_workspace_bytes(sh, cu)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    res = {}
    if scores_in is None:
        scores = torch.full((rows,), float("nan"), dtype=torch.float32, device=dev)
        raw_t = torch.full((rows, G), float("nan"), dtype=torch.float32, device=dev) if raw else None
        hs = torch.full((case.num_units, G, 2), float("nan"), dtype=torch.float64, device=dev) if stats else None
        R.tri_score(sh, cu, cp, case.k, case.k_pos, case.q_centre, case.q_absmean, case.q_R, scores,
                    raw_scores=raw_t, head_stats=hs, workspace=ws)
        res.update(scores=scores, raw=raw_t, head_stats=hs)
    else:
        scores = scores_in
        res["scores"] = scores
    kept = torch.full((max(out_rows, 1),), -1, dtype=torch.int32, device=dev)
    k_out = v_out = pos_out = None
    if compact:
        k_out = torch.zeros((max(out_rows, 1), d), dtype=torch.int16, device=dev)
        v_out = torch.zeros((max(out_rows, 1), d), dtype=torch.int16, device=dev) if case.v is not None else None
        pos_out = torch.full((max(out_rows, 1),), -1, dtype=torch.int32, device=dev)
    R.tri_select_compact(sh, cu, bu, scores, case.k if compact else None,
                         case.v if compact else None, case.k_pos if compact else None, kept,
                         k_out, v_out, pos_out, workspace=ws)
    torch.cuda.synchronize()
    res["workspace"] = ws
    res.update(kept=kept[:out_rows], k_out=None if k_out is None else k_out[:out_rows],
               v_out=None if v_out is None else v_out[:out_rows],
               pos_out=None if pos_out is None else pos_out[:out_rows])
    return res


def gpu_score_offsets(case: Case, offsets, reduce, raw=True, stats=True, raw_in_ws=False):
    """tri_score_offsets on one case.  raw_in_ws: let the library spill the
    raw scores into its workspace (raw output not requested)."""
    import rope_aware_key_amd as R
    dev = case.k.device
    sh = shape_of(case)
    G = case.shape.group
    rows = case.total_rows()
    cu = pinned(case.cu_len, np.int64)
    cp = pinned(case.cur_pos, np.int32)
    off = pinned(offsets, np.float64)
    wsb = R.tri_workspace_bytes_offsets(sh, cu, len(off), reduce)
    assert wsb > 0, R.last_error()
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    scores = torch.full((rows,), float("nan"), dtype=torch.float32, device=dev)
    raw_t = None
    if raw and not raw_in_ws:
        raw_t = torch.full((rows, G), float("nan"), dtype=torch.float32, device=dev)
    hs = torch.full((case.num_units, G, 2), float("nan"), dtype=torch.float64, device=dev) if stats else None
    R.tri_score_offsets(sh, cu, cp, case.k, case.k_pos, case.q_centre, case.q_absmean, case.q_R,
                        off, reduce, scores, raw_scores=raw_t, head_stats=hs, workspace=ws)
    torch.cuda.synchronize()
    return dict(scores=scores, raw=raw_t, head_stats=hs)


def unit_inputs(case: Case, s, l, g):
    start, n = case.unit_rows(s, l, g)
    kbits = case.k[start:start + n].cpu().numpy().view(np.uint16)
    pos = case.k_pos[start:start + n].cpu().numpy().astype(np.float64)
    G = case.shape.group
    hq = slice(g * G, (g + 1) * G)
    qc = case.q_centre[l, hq].cpu().double().numpy()
    centre = qc[..., 0] + 1j * qc[..., 1]
    absmean = case.q_absmean[l, hq].cpu().double().numpy()
    Rr = case.q_R[l, hq].cpu().double().numpy()
    return start, n, kbits, pos, centre, absmean, Rr


def oracle_unit(case: Case, s, l, g, factored=False, stats=None, offsets=None,
                reduce="mean"):
    """fp64 oracle scores of one unit. stats: optional (centre, absmean, R)
    overriding the case's fp32 statistics for this KV head's group;
    offsets/reduce: the offset set (default {2^0..2^16}) and its reduction."""
    start, n, kbits, pos, centre, absmean, Rr = unit_inputs(case, s, l, g)
    if stats is not None:
        centre, absmean, Rr = stats
    om = O.rope_omega(case.shape.head_dim, case.shape.rope_theta)
    kpost = O.bf16_bits_to_f64(kbits)
    extra = {} if offsets is None else dict(offsets=np.asarray(offsets, np.float64))
    score, S, mu, sigma = O.unit_scores(kpost, pos, float(case.cur_pos[s]), centre, absmean, Rr,
                                        om, factored=factored, reduce=reduce,
                                        layout=layout_of(case), **extra)
    return start, n, score, S, mu, sigma


def units_of(case: Case):
    L, H = case.shape.num_layers, case.shape.num_kv_heads
    return [(s, l, g) for s in range(case.num_seqs) for l in range(L) for g in range(H)]


def check_selection_exact(case: Case, res, units=None, rows_units=None):
    """kept_idx must equal the oracle's selection run on the GPU's own fp32
    scores (every unit in `units`, default all), and the compacted K, V and
    position rows must equal the input rows at those indices (units in
    `rows_units`, default the same units)."""
    scores = res["scores"].cpu().numpy()
    kept = res["kept"].cpu().numpy()
    units = units_of(case) if units is None else units
    rows_units = units if rows_units is None else rows_units
    for (s, l, g) in units:
        start, n = case.unit_rows(s, l, g)
        ostart, b = case.unit_out_rows(s, l, g)
        ref = O.select_topb(scores[start:start + n], int(case.budget[s]))
        assert len(ref) == b
        np.testing.assert_array_equal(kept[ostart:ostart + b], ref, err_msg=f"unit {(s, l, g)}")
    # small tensors come to the host once; full-size caches unit by unit
    host = {}
    for name, src_t in (("k_out", case.k), ("v_out", case.v), ("pos_out", case.k_pos)):
        out_t = res.get(name)
        if out_t is None or src_t is None:
            continue
        small = src_t.numel() * src_t.element_size() <= (256 << 20)
        host[name] = (src_t.cpu().numpy() if small else src_t,
                      out_t.cpu().numpy() if small else out_t, small)
    for (s, l, g) in rows_units:
        start, n = case.unit_rows(s, l, g)
        ostart, b = case.unit_out_rows(s, l, g)
        ref = O.select_topb(scores[start:start + n], int(case.budget[s]))
        for name, (src_a, out_a, small) in host.items():
            src = src_a[start:start + n] if small else src_a[start:start + n].cpu().numpy()
            got = out_a[ostart:ostart + b] if small else out_a[ostart:ostart + b].cpu().numpy()
            assert np.array_equal(got, O.compact_rows(src, ref)), f"{name} rows of unit {(s, l, g)}"


def check_kept_near_threshold(case: Case, res, units, factored=True):
    """The GPU's kept set of each unit against the oracle's own top-B on its
    fp64 scores: they may differ only by keys whose oracle score lies within
    1e-4 * max(1, |s_(b)|) of the oracle's b-th largest score s_(b) (the
    scores' tolerance decides those keys, not the method)."""
    kept = res["kept"].cpu().numpy()
    for (s, l, g) in units:
        ostart, b = case.unit_out_rows(s, l, g)
        if b == 0:
            continue
        _, n, ref, _, _, _ = oracle_unit(case, s, l, g, factored=factored)
        thr = np.sort(ref)[::-1][b - 1]
        diff = set(O.select_topb(ref, b).tolist()) ^ set(kept[ostart:ostart + b].tolist())
        bad = sorted(i for i in diff if abs(ref[i] - thr) > 1e-4 * max(1.0, abs(thr)))
        assert not bad, f"unit {(s, l, g)}: keys {bad[:10]} differ away from the threshold {thr}"


def gpu_score_paged(case: Case, pool, offsets=None, reduce="mean", raw=False, stats=False):
    """tri_score_paged on a case whose K sits in `pool` (synth.paged_from_case)."""
    import rope_aware_key_amd as R
    dev = case.k.device
    sh = shape_of(case)
    cu = pinned(case.cu_len, np.int64)
    cp = pinned(case.cur_pos, np.int32)
    off = None if offsets is None else pinned(offsets, np.float64)
    wsb = R.tri_workspace_bytes_paged(sh, cu, pool.page_size, 0 if offsets is None else len(off),
                                      reduce)
    assert wsb > 0, R.last_error()
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    rows, G = case.total_rows(), case.shape.group
    scores = torch.full((max(rows, 1),), float("nan"), dtype=torch.float32, device=dev)
    raw_t = torch.full((max(rows, 1), G), float("nan"), device=dev) if raw else None
    hs = torch.full((case.num_units, G, 2), float("nan"), dtype=torch.float64,
                    device=dev) if stats else None
    pages = R.make_pages(pool.table, pool.page_size, pool.num_pages, *pool.strides())
    R.tri_score_paged(sh, cu, cp, pages, pool.k, case.q_centre, case.q_absmean, case.q_R, scores,
                      offsets=off, reduce=reduce, raw_scores=raw_t, head_stats=hs, workspace=ws)
    torch.cuda.synchronize()
    return dict(scores=scores[:rows], raw=None if raw_t is None else raw_t[:rows], head_stats=hs)



def compare_units_pool(case: Case, res, units, min_bytes_free=None):
    """Every unit in `units` against the factored oracle, in worker processes
    (tests/oracle_pool.py): scores (with the z_floor bar) and (mu, sigma).
    The case and the GPU's results go to memory-mapped files the workers
    read.  Returns (worst score error, list of floors); asserts per unit."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import shutil
    import tempfile

    import checks
    import oracle_pool

    L, H, G = case.shape.num_layers, case.shape.num_kv_heads, case.shape.group
    arrays = {
        "k_pos": case.k_pos, "scores": res["scores"], "head_stats": res["head_stats"],
        "q_centre": case.q_centre, "q_absmean": case.q_absmean, "q_R": case.q_R,
    }
    need = case.k.numel() * 2 + sum(t.numel() * t.element_size() for t in arrays.values())
    base = "/dev/shm" if shutil.disk_usage("/dev/shm").free > 1.2 * need else None
    tmp = tempfile.mkdtemp(prefix="tri_oracle_", dir=base)
    try:
        files = {}
        path = os.path.join(tmp, "k.bin")
        mm = np.memmap(path, dtype=np.uint16, mode="w+", shape=tuple(case.k.shape))
        step = max(1, (256 << 20) // max(1, case.k.shape[1] * 2))
        for a in range(0, case.k.shape[0], step):
            mm[a:a + step] = case.k[a:a + step].cpu().numpy().view(np.uint16)
        mm.flush()
        del mm
        files["k"] = (path, "uint16", list(case.k.shape))
        for name, t in arrays.items():
            a = t.cpu().numpy()
            path = os.path.join(tmp, name + ".bin")
            m = np.memmap(path, dtype=a.dtype, mode="w+", shape=a.shape)
            m[...] = a
            m.flush()
            files[name] = (path, a.dtype.str, list(a.shape))
        cp = np.asarray(case.cur_pos, np.int64)
        path = os.path.join(tmp, "cur_pos.bin")
        m = np.memmap(path, dtype=np.int64, mode="w+", shape=cp.shape)
        m[...] = cp
        m.flush()
        files["cur_pos"] = (path, "<i8", list(cp.shape))
        meta = dict(G=G, d=case.shape.head_dim, theta=case.shape.rope_theta, layout=layout_of(case))
        tasks = []
        for (s, l, g) in units:
            start, n = case.unit_rows(s, l, g)
            tasks.append(((s * L + l) * H + g, s, l, g, start, n))
        nw = oracle_pool.workers()
        batch = max(1, len(tasks) // (nw * 8))
        chunks = [tasks[i:i + batch] for i in range(0, len(tasks), batch)]
        results = []
        with cf.ProcessPoolExecutor(nw, mp_context=mp.get_context("spawn"),
                                    initializer=oracle_pool.attach,
                                    initargs=(files, meta)) as ex:
            for part in ex.map(oracle_pool.score_units, chunks):
                results.extend(part)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    worst, floors = 0.0, []
    for (u, err, floor, e_mu, e_sig) in results:
        checks.note_floor(floor)
        floors.append(floor)
        assert err <= 1e-4, f"unit {u}: worst scaled score error {err:.3e} (of the 1e-4 bar)"
        assert e_mu <= 1.0 and e_sig <= 1.0, f"unit {u}: head stats off ({e_mu:.2f}, {e_sig:.2f} of their bars)"
        worst = max(worst, err)
    print(f"{len(results)} units against the oracle on {oracle_pool.workers()} processes: "
          f"worst {worst:.2e}, floors above 1e-4: {sum(f > 1e-4 for f in floors)}", flush=True)
    return worst, floors
