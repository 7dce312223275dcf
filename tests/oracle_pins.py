"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each pin is a function of an oracle module (``oracle`` or a planted-mistake
build of it) and raises AssertionError when the oracle disagrees.  The test
files call them on the real oracle; the mutation test calls them on builds
with a mistake planted in the C source and requires that some pin fails.

Pins (none re-types the oracle's formula or re-calls a routine it uses):

* library routine -- torch's scaled_dot_product_attention (fp64, CPU) for
  global attention, for frame attention as per-frame calls, for SGA on an
  explicitly augmented key set with an additive bias (count-weighted and
  unit-weight mean column), and for register attention on the compacted set
  of special tokens;
* closed forms -- zero queries give count-weighted means of the value rows;
  a hand-sized two-key example; logit ratios with one-hot values;
* invariants -- rows sum to one; frame == global at one frame; frame ==
  block-diagonal global; SGA at stride 1x1 == global; SGA with identical
  dropped keys == global (exact count weighting); diagonal present once;
  permutation equivariance over frames; Jensen bound on the mean column;
  register attention with no special tokens == frame attention;
* brute force -- the numpy matrix formulation (oracle/brute.py);
* projections -- a hand-computed linear layer (W against W^T), torch's
  linear (fp64), and the q/k/v column split with block-scaled identities.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from vga_inputs import tiny_qkv

SCALE = 0.125  # 1/sqrt(64)


def _sdpa(q, k, v, scale, mask=None):
    """torch SDPA on [T,H,d] fp64 arrays; mask: additive [T, Tk] or bool."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                         scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


def _f64(x):
    return x.astype(np.float64)


def _shape(N=2, gh=8, gw=8, S=5, H=2, d=64, seed=0):
    L = gh * gw + S
    q, k, v = tiny_qkv(N * L, H, d, seed)
    return dict(N=N, L=L, gh=gh, gw=gw, H=H, d=d), q, k, v


SGA22 = dict(stride_h=2, stride_w=2, phase_h=0, phase_w=0, diagonal=1, mean_fill=1)


# ---------------------------------------------------------------- global/frame
def pin_global_vs_sdpa(orc):
    for (N, gh, gw, S, H, seed) in [(2, 8, 8, 5, 2, 0), (3, 3, 5, 2, 3, 7)]:
        s, q, k, v = _shape(N, gh, gw, S, H, seed=seed)
        o = orc.attention(orc.MODE_GLOBAL, q, k, v, s["N"], s["L"], gh, gw, SCALE)
        ref = _sdpa(_f64(q), _f64(k), _f64(v), SCALE)
        assert np.max(np.abs(o - ref)) < 1e-12, "global != SDPA"


def pin_frame_vs_sdpa(orc):
    s, q, k, v = _shape(3, 4, 6, 3, 2, seed=3)
    L = s["L"]
    o = orc.attention(orc.MODE_FRAME, q, k, v, 3, L, 4, 6, SCALE)
    for f in range(3):
        sl = slice(f * L, (f + 1) * L)
        ref = _sdpa(_f64(q[sl]), _f64(k[sl]), _f64(v[sl]), SCALE)
        assert np.max(np.abs(o[sl] - ref)) < 1e-12, "frame != per-frame SDPA"
    # block-diagonal mask over all tokens (frame attention is global attention
    # restricted to each frame's own tokens)
    fr = np.arange(3 * L) // L
    mask = np.where(fr[:, None] == fr[None, :], 0.0, -np.inf)
    ref = _sdpa(_f64(q), _f64(k), _f64(v), SCALE, mask)
    assert np.max(np.abs(o - ref)) < 1e-12, "frame != block-diagonal global"


def pin_frame_equals_global_one_frame(orc):
    s, q, k, v = _shape(1, 5, 5, 3, 2, seed=4)
    a = orc.attention(orc.MODE_FRAME, q, k, v, 1, s["L"], 5, 5, SCALE)
    b = orc.attention(orc.MODE_GLOBAL, q, k, v, 1, s["L"], 5, 5, SCALE)
    assert np.max(np.abs(a - b)) < 1e-14


def pin_two_key_closed_form(orc):
    # one head, two tokens in one frame; logits 0 and ln 3 -> weights 1/4, 3/4
    d = 64
    q = np.zeros((2, 1, d), np.float32)
    k = np.zeros((2, 1, d), np.float32)
    v = np.zeros((2, 1, d), np.float32)
    q[:, 0, 0] = 1.0
    k[1, 0, 0] = math.log(3.0)
    v[0, 0, 1], v[1, 0, 1] = 4.0, 8.0
    v[0, 0, 2], v[1, 0, 2] = -2.0, 2.0
    kl = np.float64(np.float32(math.log(3.0)))       # ln 3 as stored in fp32
    w1 = math.exp(kl) / (1.0 + math.exp(kl))
    for mode in (orc.MODE_GLOBAL, orc.MODE_FRAME):
        o = orc.attention(mode, q, k, v, 1, 2, 0, 0, 1.0)
        assert abs(o[0, 0, 1] - (4.0 * (1 - w1) + 8.0 * w1)) < 1e-14
        assert abs(o[1, 0, 2] - (-2.0 * (1 - w1) + 2.0 * w1)) < 1e-14
        assert abs(o[0, 0, 1] - 7.0) < 1e-6                # 4/4 + 3*8/4
        assert np.all(o[:, 0, 3:] == 0.0) and np.all(o[:, 0, 0] == 0.0)


def pin_zero_query_means(orc):
    # q = 0: every logit 0, so each column weighs 1 (the mean column |D|)
    s, q, k, v = _shape(2, 4, 4, 3, 2, seed=5)
    N, L, gh, gw = s["N"], s["L"], 4, 4
    q = np.zeros_like(q)
    v64 = _f64(v)
    og = orc.attention(orc.MODE_GLOBAL, q, k, v, N, L, gh, gw, SCALE)
    assert np.max(np.abs(og - v64.mean(axis=0)[None])) < 1e-13
    of = orc.attention(orc.MODE_FRAME, q, k, v, N, L, gh, gw, SCALE)
    for f in range(N):
        m = v64[f * L:(f + 1) * L].mean(axis=0)
        assert np.max(np.abs(of[f * L:(f + 1) * L] - m[None])) < 1e-13
    _, keep = orc.select(N, L, gh, gw, 2, 2, 0, 0)
    keep = keep.astype(bool)
    T = N * L
    for diag in (0, 1):
        for mean in (0, 1, 2):
            p = dict(SGA22, diagonal=diag, mean_fill=mean)
            o = orc.attention(orc.MODE_SGA, q, k, v, N, L, gh, gw, SCALE, p)
            for i in range(T):
                cols = v64[keep].sum(axis=0)
                n = keep.sum()
                if mean == 1:                  # |D| copies of vmean = sum of dropped
                    cols = cols + v64[~keep].sum(axis=0)
                    n = T
                elif mean == 2:                # one column holding the mean
                    cols = cols + v64[~keep].mean(axis=0)
                    n = n + 1
                if diag and not keep[i]:
                    cols = cols + v64[i]
                    n = n + 1
                assert np.max(np.abs(o[i] - cols / n)) < 1e-13, (diag, mean, i)


def pin_rows_stochastic_and_ratios(orc):
    # one-hot values (d == T) turn the output rows into the probability rows
    N, gh, gw, S, H = 1, 4, 4, 2, 2
    L = gh * gw + S
    T = N * L
    rng = np.random.default_rng(11)
    q = rng.standard_normal((T, H, T)).astype(np.float32)
    k = rng.standard_normal((T, H, T)).astype(np.float32)
    v = np.zeros((T, H, T), np.float32)
    for h in range(H):
        v[:, h, :] = np.eye(T, dtype=np.float32)
    sc = 1.0 / math.sqrt(T)
    p = orc.attention(orc.MODE_GLOBAL, q, k, v, N, L, gh, gw, sc)
    assert np.max(np.abs(p.sum(axis=2) - 1.0)) < 1e-13
    z = sc * np.einsum("ihe,jhe->hij", _f64(q), _f64(k))
    for h in range(H):
        for i in (0, 5, T - 1):
            # a zero probability (a planted mistake) gives -inf and fails
            with np.errstate(divide="ignore"):
                lr = np.log(p[i, h, :] / p[i, h, 0])
            assert np.max(np.abs(lr - (z[h, i] - z[h, i, 0]))) < 1e-10
    # SGA rows also sum to one over subset + diagonal + mean (shared softmax)
    s = dict(SGA22)
    ps = orc.attention(orc.MODE_SGA, q, k, v, N, L, gh, gw, sc, s)
    assert np.max(np.abs(ps.sum(axis=2) - 1.0)) < 1e-13


def pin_vs_brute(orc):
    from oracle import brute
    for (N, gh, gw, S, H, seed) in [(2, 8, 8, 5, 2, 0), (3, 5, 7, 1, 1, 9)]:
        s, q, k, v = _shape(N, gh, gw, S, H, seed=seed)
        L = s["L"]
        for mode, name in ((orc.MODE_GLOBAL, "global"), (orc.MODE_FRAME, "frame"),
                           (orc.MODE_REGISTER, "register")):
            o = orc.attention(mode, q, k, v, N, L, gh, gw, SCALE)
            ref = brute.attention(name, _f64(q), _f64(k), _f64(v), N, L, gh, gw, SCALE)
            assert np.max(np.abs(o - ref)) < 1e-12, name
        for p in (SGA22, dict(stride_h=3, stride_w=2, phase_h=1, phase_w=1,
                              diagonal=1, mean_fill=1),
                  dict(stride_h=2, stride_w=3, phase_h=1, phase_w=0,
                       diagonal=0, mean_fill=1),
                  dict(stride_h=3, stride_w=3, phase_h=2, phase_w=1,
                       diagonal=1, mean_fill=0),
                  dict(SGA22, mean_fill=2)):
            o = orc.attention(orc.MODE_SGA, q, k, v, N, L, gh, gw, SCALE, p)
            ref = brute.attention("sga", _f64(q), _f64(k), _f64(v), N, L, gh, gw,
                                  SCALE, p)
            assert np.max(np.abs(o - ref)) < 1e-12, p


# ------------------------------------------------------------------------- SGA
def pin_sga_vs_sdpa_augmented(orc):
    s, q, k, v = _shape(2, 6, 5, 3, 2, seed=12)
    N, L, gh, gw = s["N"], s["L"], 6, 5
    T = N * L
    p = dict(stride_h=2, stride_w=2, phase_h=1, phase_w=0, diagonal=1, mean_fill=1)
    # key set: every token, then the mean column; bias masks and weights them
    keep = np.zeros(T, bool)
    for f in range(N):
        for u in range(L):
            if u >= gh * gw or ((u // gw) % 2 == 1 and (u % gw) % 2 == 0):
                keep[f * L + u] = True
    nd = int((~keep).sum())
    k64, v64 = _f64(k), _f64(v)
    ka = np.concatenate([k64, k64[~keep].mean(axis=0)[None]], axis=0)
    va = np.concatenate([v64, v64[~keep].mean(axis=0)[None]], axis=0)
    bias = np.full((T, T + 1), -np.inf)
    bias[:, :T][:, keep] = 0.0
    bias[np.arange(T), np.arange(T)] = 0.0
    bias[:, T] = math.log(nd)
    ref = _sdpa(_f64(q), ka, va, SCALE, bias)
    o = orc.attention(orc.MODE_SGA, q, k, v, N, L, gh, gw, SCALE, p)
    assert np.max(np.abs(o - ref)) < 1e-12


def pin_sga_unit_weight_vs_sdpa(orc):
    # unit-weight mean column: the same augmented key set with bias 0 (one
    # column) instead of ln|D|
    s, q, k, v = _shape(2, 5, 6, 2, 2, seed=14)
    N, L, gh, gw = s["N"], s["L"], 5, 6
    T = N * L
    p = dict(stride_h=2, stride_w=3, phase_h=0, phase_w=1, diagonal=1, mean_fill=2)
    keep = np.zeros(T, bool)
    for f in range(N):
        for u in range(L):
            if u >= gh * gw or ((u // gw) % 2 == 0 and (u % gw) % 3 == 1):
                keep[f * L + u] = True
    k64, v64 = _f64(k), _f64(v)
    ka = np.concatenate([k64, k64[~keep].mean(axis=0)[None]], axis=0)
    va = np.concatenate([v64, v64[~keep].mean(axis=0)[None]], axis=0)
    bias = np.full((T, T + 1), -np.inf)
    bias[:, :T][:, keep] = 0.0
    bias[np.arange(T), np.arange(T)] = 0.0
    bias[:, T] = 0.0
    ref = _sdpa(_f64(q), ka, va, SCALE, bias)
    o = orc.attention(orc.MODE_SGA, q, k, v, N, L, gh, gw, SCALE, p)
    assert np.max(np.abs(o - ref)) < 1e-12


def pin_sga_stride1_is_global(orc):
    s, q, k, v = _shape(2, 4, 5, 2, 2, seed=13)
    N, L = s["N"], s["L"]
    g = orc.attention(orc.MODE_GLOBAL, q, k, v, N, L, 4, 5, SCALE)
    for diag in (0, 1):
        p = dict(stride_h=1, stride_w=1, phase_h=0, phase_w=0, diagonal=diag,
                 mean_fill=1)
        o = orc.attention(orc.MODE_SGA, q, k, v, N, L, 4, 5, SCALE, p)
        assert np.max(np.abs(o - g)) < 1e-13


def pin_sga_identical_dropped_keys(orc):
    # all dropped tokens share one key k* and value v*: |D| exp(s q.k*) equals
    # the exact sum over the dropped columns, so SGA == global when diagonal is
    # off, and == global plus one more (k*, v*) column when it is on.
    N, gh, gw, S, H = 2, 6, 6, 3, 2
    L = gh * gw + S
    T = N * L
    q, k, v = tiny_qkv(T, H, 64, 21)
    _, keep = orc.select(N, L, gh, gw, 3, 2, 1, 0)
    keep = keep.astype(bool)
    rng = np.random.default_rng(22)
    kstar = rng.standard_normal((H, 64)).astype(np.float32)
    vstar = rng.standard_normal((H, 64)).astype(np.float32)
    k[~keep] = kstar
    v[~keep] = vstar
    p = dict(stride_h=3, stride_w=2, phase_h=1, phase_w=0, diagonal=0, mean_fill=1)
    o = orc.attention(orc.MODE_SGA, q, k, v, N, L, gh, gw, SCALE, p)
    g = orc.attention(orc.MODE_GLOBAL, q, k, v, N, L, gh, gw, SCALE)
    assert np.max(np.abs(o - g)) < 1e-12
    p["diagonal"] = 1
    o = orc.attention(orc.MODE_SGA, q, k, v, N, L, gh, gw, SCALE, p)
    ka = np.concatenate([_f64(k), _f64(kstar)[None]], axis=0)
    va = np.concatenate([_f64(v), _f64(vstar)[None]], axis=0)
    bias = np.zeros((T, T + 1))
    bias[keep, T] = -np.inf                 # kept queries get no diagonal extra
    ref = _sdpa(_f64(q), ka, va, SCALE, bias)
    assert np.max(np.abs(o - ref)) < 1e-12


def pin_sga_diagonal_once(orc):
    # one-hot values expose the weight of every column; with the mean off the
    # row is a softmax over kept columns plus the own column iff dropped.
    N, gh, gw, S, H = 1, 4, 4, 2, 1
    L = gh * gw + S
    T = N * L
    rng = np.random.default_rng(31)
    q = rng.standard_normal((T, H, T)).astype(np.float32)
    k = rng.standard_normal((T, H, T)).astype(np.float32)
    v = np.eye(T, dtype=np.float32)[:, None, :]
    sc = 1.0 / math.sqrt(T)
    _, keep = orc.select(N, L, gh, gw, 2, 2, 0, 0)
    keep = keep.astype(bool)
    p = dict(stride_h=2, stride_w=2, phase_h=0, phase_w=0, diagonal=1, mean_fill=0)
    o = orc.attention(orc.MODE_SGA, q, k, v, N, L, gh, gw, sc, p)[:, 0, :]
    z = sc * _f64(q[:, 0, :]) @ _f64(k[:, 0, :]).T
    for i in range(T):
        cols = keep.copy()
        cols[i] = True
        w = np.where(cols, np.exp(z[i] - z[i][cols].max()), 0.0)
        assert np.max(np.abs(o[i] - w / w.sum())) < 1e-13, i
        # the own column appears exactly once: its weight equals one share
        assert abs(o[i, i] - w[i] / w.sum()) < 1e-13


def pin_sga_jensen(orc):
    # the mean column never outweighs the exact dropped mass:
    # |D| exp(s q.kmean) <= sum_{j in D} exp(s q.k_j)  (convexity of exp)
    s, q, k, v = _shape(2, 6, 6, 3, 2, seed=41)
    N, L, gh, gw = s["N"], s["L"], 6, 6
    km, vm, nd = orc.dropped_mean(k, v, N, L, gh, gw, 2, 2, 0, 0)
    _, keep = orc.select(N, L, gh, gw, 2, 2, 0, 0)
    drop = ~keep.astype(bool)
    assert nd == drop.sum()
    k64, v64 = _f64(k), _f64(v)
    assert np.max(np.abs(km - k64[drop].mean(axis=0))) < 1e-14
    assert np.max(np.abs(vm - v64[drop].mean(axis=0))) < 1e-14
    q64 = _f64(q)
    for h in range(2):
        lhs = nd * np.exp(SCALE * q64[:, h] @ km[h])
        rhs = np.exp(SCALE * q64[:, h] @ k64[drop, h].T).sum(axis=1)
        assert np.all(lhs <= rhs * (1 + 1e-12))


def pin_permutation_equivariance(orc):
    s, q, k, v = _shape(3, 4, 4, 2, 2, seed=51)
    N, L = s["N"], s["L"]
    perm = np.array([2, 0, 1])
    idx = (perm[:, None] * L + np.arange(L)[None]).reshape(-1)
    for mode, p in ((orc.MODE_GLOBAL, None), (orc.MODE_FRAME, None),
                    (orc.MODE_SGA, SGA22), (orc.MODE_REGISTER, None)):
        a = orc.attention(mode, q, k, v, N, L, 4, 4, SCALE, p)
        b = orc.attention(mode, q[idx], k[idx], v[idx], N, L, 4, 4, SCALE, p)
        assert np.max(np.abs(a[idx] - b)) < 1e-12, mode


def pin_row_subset(orc):
    s, q, k, v = _shape(2, 8, 8, 5, 2, seed=61)
    N, L = s["N"], s["L"]
    rows = np.array([137, 0, 70, 69, 5])
    for mode, p in ((orc.MODE_GLOBAL, None), (orc.MODE_FRAME, None),
                    (orc.MODE_SGA, SGA22), (orc.MODE_REGISTER, None)):
        full = orc.attention(mode, q, k, v, N, L, 8, 8, SCALE, p)
        part = orc.attention(mode, q, k, v, N, L, 8, 8, SCALE, p, rows=rows)
        assert np.array_equal(full[rows], part)


# ------------------------------------------------------------ register attention
def pin_register_vs_sdpa(orc):
    # special rows: SDPA over the special tokens of all frames, gathered into a
    # compact set; patch rows: SDPA over their own frame
    for (N, gh, gw, S, H, seed) in [(3, 4, 5, 3, 2, 71), (2, 8, 8, 5, 2, 72)]:
        s, q, k, v = _shape(N, gh, gw, S, H, seed=seed)
        L = s["L"]
        T = N * L
        o = orc.attention(orc.MODE_REGISTER, q, k, v, N, L, gh, gw, SCALE)
        sp = np.array([f * L + u for f in range(N) for u in range(gh * gw, L)])
        ref = _sdpa(_f64(q[sp]), _f64(k[sp]), _f64(v[sp]), SCALE)
        assert np.max(np.abs(o[sp] - ref)) < 1e-12, "special rows"
        for f in range(N):
            sl = slice(f * L, f * L + gh * gw)
            fr = slice(f * L, (f + 1) * L)
            ref = _sdpa(_f64(q[sl]), _f64(k[fr]), _f64(v[fr]), SCALE)
            assert np.max(np.abs(o[sl] - ref)) < 1e-12, "patch rows"
        assert len(sp) == N * S and T == N * (gh * gw + S)


def pin_register_special_cases(orc):
    # no special tokens: register attention is frame attention
    s, q, k, v = _shape(3, 3, 4, 0, 2, seed=73)
    a = orc.attention(orc.MODE_REGISTER, q, k, v, 3, s["L"], 3, 4, SCALE)
    b = orc.attention(orc.MODE_FRAME, q, k, v, 3, s["L"], 3, 4, SCALE)
    assert np.max(np.abs(a - b)) < 1e-14
    # zero queries: a special row is the mean value of every special token, a
    # patch row the mean value of its frame
    s, q, k, v = _shape(3, 3, 3, 2, 2, seed=74)
    N, L = 3, s["L"]
    q = np.zeros_like(q)
    v64 = _f64(v)
    o = orc.attention(orc.MODE_REGISTER, q, k, v, N, L, 3, 3, SCALE)
    special = (np.arange(N * L) % L) >= 9
    for i in range(N * L):
        f = i // L
        m = v64[special].mean(axis=0) if special[i] else v64[f * L:(f + 1) * L].mean(axis=0)
        assert np.max(np.abs(o[i] - m)) < 1e-13, i


# ------------------------------------------------------------------- selection
def kept_per_frame_closed_form(gh, gw, S, sh, sw, oh, ow):
    """S + ceil((gh-oh)/sh) * ceil((gw-ow)/sw): lattice points r = oh + a*sh."""
    return S + (-(-(gh - oh) // sh)) * (-(-(gw - ow) // sw))


def pin_selection_counts(orc):
    for (gh, gw, S, sh, sw, oh, ow) in [(8, 8, 5, 2, 2, 0, 0), (37, 37, 5, 2, 2, 0, 0),
                                        (37, 37, 5, 3, 3, 1, 1), (5, 7, 2, 3, 2, 2, 1),
                                        (6, 4, 0, 1, 1, 0, 0), (3, 3, 1, 4, 4, 3, 3)]:
        L = gh * gw + S
        idx, mask = orc.select(3, L, gh, gw, sh, sw, oh, ow)
        kpf = kept_per_frame_closed_form(gh, gw, S, sh, sw, oh, ow)
        assert len(idx) == 3 * kpf and int(mask.sum()) == 3 * kpf


def pin_selection_windows(orc):
    # every full sh x sw window of the grid holds exactly one kept patch, at
    # window offset (oh, ow); specials are always kept; the list is ascending
    for (gh, gw, S, sh, sw, oh, ow) in [(8, 8, 5, 2, 2, 0, 0), (9, 7, 3, 3, 3, 1, 1),
                                        (7, 10, 2, 2, 3, 1, 2), (37, 37, 5, 3, 3, 1, 1)]:
        L = gh * gw + S
        N = 2
        idx, mask = orc.select(N, L, gh, gw, sh, sw, oh, ow)
        assert np.all(np.diff(idx) > 0)
        assert np.array_equal(np.flatnonzero(mask), idx)
        for f in range(N):
            m = mask[f * L:(f + 1) * L]
            assert np.all(m[gh * gw:] == 1)
            g = m[: gh * gw].reshape(gh, gw)
            for r0 in range(0, gh - sh + 1, sh):
                for c0 in range(0, gw - sw + 1, sw):
                    win = g[r0:r0 + sh, c0:c0 + sw]
                    assert win.sum() == 1 and win[oh, ow] == 1


def pin_schedule(orc):
    s = orc.schedule(24, 8, True)
    assert list(s) == [orc.MODE_FRAME] * 8 + [orc.MODE_SGA] * 16
    s = orc.schedule(5, 2, False)
    assert list(s) == [orc.MODE_FRAME] * 2 + [orc.MODE_GLOBAL] * 3
    assert list(orc.schedule(3, 3, True)) == [orc.MODE_FRAME] * 3
    assert list(orc.schedule(0, 0, True)) == []
    # every 4th slot (a quarter) runs register attention, early slots excepted
    F, G, S_, R = orc.MODE_FRAME, orc.MODE_GLOBAL, orc.MODE_SGA, orc.MODE_REGISTER
    assert list(orc.schedule_register(8, 0, 4, False)) == [G, G, G, R, G, G, G, R]
    r = orc.schedule_register(24, 8, 4, True)
    assert list(r) == [F] * 8 + [S_, S_, S_, R] * 4
    assert int((orc.schedule_register(24, 0, 4, False) == R).sum()) == 6
    assert list(orc.schedule_register(6, 2, 0, True)) == list(orc.schedule(6, 2, True))


# ------------------------------------------------- projections around a layer
def _bf16_bits(a):
    """float32 values that bf16 holds exactly -> raw bf16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def pin_linear_worked_example(orc):
    # hand-computed: y = x W^T + b with W's rows the output features
    x = np.array([[1, 2, 3], [4, 5, 6]], np.float32)
    w = np.array([[1, 0, -1], [2, 1, 0]], np.float32)
    b = np.array([0.5, -1], np.float32)
    assert np.array_equal(orc.linear(x, w, b), [[-1.5, 3.0], [-1.5, 12.0]])
    # a square, non-symmetric W tells W from W^T
    x = np.array([[1, 2]], np.float32)
    w = np.array([[0, 1], [3, 0]], np.float32)
    assert np.array_equal(orc.linear(x, w), [[2.0, 3.0]])
    assert np.array_equal(orc.linear(_bf16_bits(x), _bf16_bits(w)), [[2.0, 3.0]])


def pin_linear_vs_torch(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 128)).astype(np.float32)
    w = rng.standard_normal((96, 128)).astype(np.float32)
    b = rng.standard_normal(96).astype(np.float32)
    ref = torch.nn.functional.linear(torch.from_numpy(_f64(x)), torch.from_numpy(_f64(w)),
                                     torch.from_numpy(_f64(b))).numpy()
    assert np.max(np.abs(orc.linear(x, w, b) - ref)) < 1e-12
    ref = torch.nn.functional.linear(torch.from_numpy(_f64(x)), torch.from_numpy(_f64(w))).numpy()
    assert np.max(np.abs(orc.linear(x, w) - ref)) < 1e-12


def pin_qkv_split(orc):
    # W = [I; 2I; 3I] and b = [0; 1; 2] (per block) give q = x, k = 2x + 1,
    # v = 3x + 2, each as [M, H, 64] with feature 64h + e in head h, dim e
    H, M = 2, 5
    C = 64 * H
    rng = np.random.default_rng(6)
    x = rng.integers(-8, 9, size=(M, C)).astype(np.float32)
    eye = np.eye(C, dtype=np.float32)
    w = np.concatenate([eye, 2 * eye, 3 * eye])
    b = np.repeat(np.arange(3, dtype=np.float32), C)
    for conv in (lambda a: a, _bf16_bits):
        q, k, v = orc.qkv_proj(conv(x), conv(w), conv(b), H)
        xr = x.reshape(M, H, 64)
        assert np.array_equal(q, xr) and np.array_equal(k, 2 * xr + 1)
        assert np.array_equal(v, 3 * xr + 2)


ALL_PINS = [v for kname, v in sorted(globals().items()) if kname.startswith("pin_")]
