"""The decode-loop driver (tri_decode_*) against the oracle's decode loop.

At every prune, the GPU's scores are held to the tri_score bar against the
oracle (|gpu - ref| <= 1e-4 * max(1, |ref|) on the keys that compete; the
protected keys read +inf), and the oracle then keeps select_protected of
the GPU's own scores, as the parity tests do for the top-B.  The caches
(K, V, positions, lengths) must match the oracle's bit for bit after every
step checked.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import check_scores, dev_read, half_split, layout_of, shape_of

pytestmark = pytest.mark.gpu

DEV = "cuda"


class Stream:
    """One synthetic decode run: sequence s has n_pre[s] prompt keys and
    `steps` generated ones, all drawn at positions 0, 1, 2, ..."""

    def __init__(self, shape, n_pre, steps, seed, layout="interleaved"):
        self.shape, self.n_pre, self.steps = shape, list(n_pre), steps
        lens = tuple(n + steps for n in n_pre)
        self.case = synth.build_case("decode", shape, lens, tuple([1] * len(lens)), device=DEV,
                                     seed=seed)
        if layout == "half":
            self.case = half_split(self.case)
        self.S = len(n_pre)
        self.LH = shape.num_layers * shape.num_kv_heads

    def unit_start(self, s, lg):
        c = self.case
        return self.LH * int(c.cu_len[s]) + lg * c.seq_len(s)

    def prefill_rows(self):
        idx = [np.arange(self.unit_start(s, lg), self.unit_start(s, lg) + self.n_pre[s])
               for s in range(self.S) for lg in range(self.LH)]
        return torch.as_tensor(np.concatenate(idx), device=DEV)

    def token_rows(self, t):
        return torch.as_tensor([self.unit_start(s, lg) + self.n_pre[s] + t
                                for s in range(self.S) for lg in range(self.LH)], device=DEV)

    def stats(self, l, g):
        G = self.shape.group
        hq = slice(g * G, (g + 1) * G)
        qc = self.case.q_centre[l, hq].cpu().double().numpy()
        return (qc[..., 0] + 1j * qc[..., 1], self.case.q_absmean[l, hq].cpu().double().numpy(),
                self.case.q_R[l, hq].cpu().double().numpy())


def _oracle_units(st, rows_k, rows_v, rows_p):
    units = {}
    o = 0
    for s in range(st.S):
        for lg in range(st.LH):
            n = st.n_pre[s]
            units[s, lg] = O.DecodeUnit(rows_k[o:o + n], rows_v[o:o + n], rows_p[o:o + n])
            o += n
    return units


def _prune_oracle(st, dec, units, s, B, sink, recent, p_q, check=True):
    """Apply the prune the GPU just ran on sequence s to the oracle units,
    with the GPU's scores, after checking them against the oracle's."""
    vw = dec.view()
    om = O.rope_omega(st.shape.head_dim, st.shape.rope_theta)
    L, H = st.shape.num_layers, st.shape.num_kv_heads
    for lg in range(st.LH):
        u = units[s, lg]
        n = len(u)
        gpu = dev_read(vw["scores"][s] + lg * vw["scores_stride"][s] * 4, n, np.float32)
        prot = O.protected_mask(n, sink, recent)
        assert np.all(np.isposinf(gpu[prot]))
        if check:
            ref = u.scores(*st.stats(lg // H, lg % H), om, factored=True, p_q=p_q,
                           layout=layout_of(st.case))
            check_scores(gpu[~prot], ref[~prot], f"prune of unit {(s, lg)}")
        u.prune(O.select_protected(gpu, B, sink, recent))


def _check_cache(st, dec, units):
    vw = dec.view()
    d, C = st.shape.head_dim, vw["unit_stride"]
    for s in range(st.S):
        for lg in range(st.LH):
            u = units[s, lg]
            n = len(u)
            assert vw["len"][s] == n, (s, vw["len"][s], n)
            k = dev_read(vw["k"][s] + lg * C * d * 2, n * d, np.uint16).reshape(n, d)
            v = dev_read(vw["v"][s] + lg * C * d * 2, n * d, np.uint16).reshape(n, d)
            p = dev_read(vw["pos"][s] + lg * C * 4, n, np.int32)
            np.testing.assert_array_equal(p, u.pos, err_msg=f"positions of unit {(s, lg)}")
            assert np.array_equal(k, u.k), f"K of unit {(s, lg)}"
            assert np.array_equal(v, u.v), f"V of unit {(s, lg)}"


def _run(shape, n_pre, steps, B, interval, sink, recent, seed, check_every=1, check_scores=True,
         layout="interleaved"):
    import rope_aware_key_amd as R
    st = Stream(shape, n_pre, steps, seed, layout)
    c = st.case
    C = B + interval
    dec = R.Decode(shape_of(c), st.S, B, interval, c.q_centre, c.q_absmean, c.q_R,
                   protect_sink=sink, protect_recent=recent)
    try:
        pr = st.prefill_rows()
        k0, v0, p0 = c.k[pr].contiguous(), c.v[pr].contiguous(), c.k_pos[pr].contiguous()
        cu = np.concatenate([[0], np.cumsum(st.n_pre)]).astype(np.int64)
        cur = [st.n_pre[s] - 1 for s in range(st.S)]   # newest prompt key
        dec.prefill(cu, cur, k0, v0, p0)
        units = _oracle_units(st, k0.cpu().numpy().view(np.uint16), v0.cpu().numpy().view(np.uint16),
                              p0.cpu().numpy())
        prunes = 0
        for s in range(st.S):
            if st.n_pre[s] >= C:
                _prune_oracle(st, dec, units, s, B, sink, recent, cur[s], check_scores)
                prunes += 1
        _check_cache(st, dec, units)
        for t in range(steps):
            tr = st.token_rows(t)
            kn, vn, pn = c.k[tr].contiguous(), c.v[tr].contiguous(), c.k_pos[tr].cpu().numpy()
            pos_new = pn.reshape(st.S, st.LH)[:, 0]
            dec.append(kn, vn, pos_new)
            kb, vb = kn.cpu().numpy().view(np.uint16), vn.cpu().numpy().view(np.uint16)
            for s in range(st.S):
                for lg in range(st.LH):
                    units[s, lg].append(kb[s * st.LH + lg], vb[s * st.LH + lg], pos_new[s])
                if len(units[s, 0]) == C:
                    _prune_oracle(st, dec, units, s, B, sink, recent, pos_new[s], check_scores)
                    prunes += 1
            if (t + 1) % check_every == 0 or t == steps - 1:
                _check_cache(st, dec, units)
        assert dec.view()["prunes"] == prunes
        return prunes
    finally:
        dec.close()


@pytest.mark.parametrize("sink,recent", [(0, 0), (2, 5), (4, 0), (0, 9)])
def test_decode_loop_small(sink, recent):
    """G = 2, d = 128, three sequences: one below the trigger, one a key short
    of it, one pruned at prefill; 30 appends prune each of them at
    different steps.  Caches checked after every append."""
    shape = synth.Shape(128, 4, 2, 2)
    prunes = _run(shape, [30, 47, 60], 30, B=40, interval=8, sink=sink, recent=recent,
                  seed=3 + sink + recent)
    assert prunes >= 6


def test_decode_loop_generic_path_and_ragged():
    """head_dim 48 takes the VALU score path; five sequences of different
    lengths, an interval of 1 (a prune after every append once full)."""
    shape = synth.Shape(48, 6, 2, 1)
    _run(shape, [0, 5, 19, 20, 33], 12, B=18, interval=1, sink=1, recent=2, seed=11)


@pytest.mark.parametrize("d", [128, 48])
def test_decode_loop_half_split(d):
    """Keys stored half split (MFMA path at d = 128, VALU path at 48)."""
    shape = synth.Shape(d, 4, 2, 1)
    prunes = _run(shape, [20, 45], 24, B=30, interval=6, sink=2, recent=3, seed=17,
                  layout="half")
    assert prunes >= 4


def test_decode_loop_protected_fill_budget():
    """sink + recent = budget: the cache is always the first `sink` and the
    latest `recent` keys, whatever the scores."""
    shape = synth.Shape(64, 8, 1, 1)
    _run(shape, [10, 50], 25, B=12, interval=4, sink=5, recent=7, seed=5, check_scores=False)


@pytest.mark.timeout(600)
def test_decode_loop_decode_window_shape():
    """The decode-window shape (G = 4, d = 128, budget 3072, interval 128) on
    two sequences and two layers: a prompt of 3200 keys pruned at prefill,
    then 256 appends and two more prunes; caches checked after each prune."""
    shape = synth.Shape(128, 32, 8, 2)
    _run(shape, [3200, 3100], 256, B=3072, interval=128, sink=4, recent=64, seed=2,
         check_every=128)


def test_decode_loop_many_sequences_staged_append():
    """130 sequences, past the 128 whose append items ride in the kernel
    arguments: the items go through the staging copy instead.  Short
    prompts of different lengths, a prune every 4 appends."""
    shape = synth.Shape(64, 2, 1, 1)
    g = np.random.default_rng(41)
    n_pre = [int(x) for x in g.integers(0, 14, size=130)]
    prunes = _run(shape, n_pre, 9, B=8, interval=4, sink=1, recent=2, seed=41, check_every=3)
    assert prunes >= 130


@pytest.mark.timeout(600)
def test_decode_loop_long_context_split_select():
    """Prompts of 40000 and 36100 keys with a budget of 36000: every prune
    selects over units past 35840 keys, so the split select runs inside the
    loop (at prefill and after 64 appends), with sinks and a recent window."""
    shape = synth.Shape(64, 2, 1, 1)
    prunes = _run(shape, [40000, 36100], 70, B=36000, interval=64, sink=4, recent=32, seed=29,
                  check_every=35)
    assert prunes == 4


@pytest.mark.parametrize("seed", range(12))
def test_decode_loop_random(seed):
    """Seeded random decode runs: head_dim, group, layers, prompt lengths,
    budget, interval, protection and RoPE layout drawn per case; caches
    checked against the oracle after every append."""
    g = np.random.default_rng([92, seed])
    d = int(g.integers(1, 9)) * 32 if g.random() < 0.5 else int(g.integers(1, 33)) * 8
    G, Hkv, L = int(g.integers(1, 9)), int(g.integers(1, 3)), int(g.integers(1, 3))
    B = int(g.integers(4, 48))
    interval = int(g.integers(1, 12))
    sink = int(g.integers(0, 4))
    recent = int(g.integers(0, max(1, B - sink - 1)))
    n_pre = [int(x) for x in g.integers(0, B + interval + 10, size=int(g.integers(1, 4)))]
    layout = "half" if g.random() < 0.5 else "interleaved"
    print(f"decode case {seed}: d={d} G={G} Hkv={Hkv} L={L} B={B} interval={interval} "
          f"sink={sink} recent={recent} prompts={n_pre} {layout}", flush=True)
    shape = synth.Shape(d, G * Hkv, Hkv, L)
    _run(shape, n_pre, int(g.integers(5, 25)), B=B, interval=interval, sink=sink, recent=recent,
         seed=seed, layout=layout)
