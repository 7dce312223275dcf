"""Brute-force numpy formulation of the same attention definitions -- TEST
INFRASTRUCTURE ONLY, for tiny inputs (it materialises the full logit matrix).

It is written independently of ``vga_oracle.c``: instead of per-row column
lists it builds, per head, the whole (T x T) logit matrix, masks it, appends
the mean-fill column and takes a row softmax -- the "one shared softmax"
reading of "AVGGT: Rethinking Global Attention for Accelerating VGGT",
technical summary section 3, step two (SGA).

Register attention ("VGGT-Omega" notes, section 2, Register Attention) is
the same matrix with a mask that lets special tokens see only special
tokens (of every frame) and patch tokens see only their own frame.

Inputs are float64 arrays [T, H, d].
"""
from __future__ import annotations

import numpy as np


def _grid_keep_mask(N, L, gh, gw, sh, sw, oh, ow):
    """Kept-token mask built on the 2D patch grid, frame by frame."""
    frame = np.ones(L, dtype=bool)             # specials stay (not grid points)
    grid = np.zeros((gh, gw), dtype=bool)
    grid[oh::sh, ow::sw] = True                 # one sample per sh x sw window
    frame[: gh * gw] = grid.reshape(-1)
    return np.tile(frame, N)


def _softmax_rows(z):
    z = z - z.max(axis=-1, keepdims=True)
    w = np.exp(z)
    return w / w.sum(axis=-1, keepdims=True)


def attention(mode, q, k, v, N, L, gh, gw, scale, sga=None, mean_copies=False):
    """mode: 'frame' | 'global' | 'sga' | 'register'.  Returns [T, H, d]
    float64.

    mean_copies=True realises the count-weighted mean column literally as |D|
    identical (kmean, vmean) columns with no log term, instead of one column
    with logit + ln|D| -- the two must agree.  sga["mean_fill"] == 2 is the
    unit-weight column (logit without ln|D|)."""
    T, H, d = q.shape
    assert T == N * L
    z = scale * np.einsum("ihe,jhe->hij", q, k)          # [H, T, T]
    allowed = np.ones((T, T), dtype=bool)
    vals = [v.transpose(1, 0, 2)]                         # [H, T, d]
    extra_logits = None
    if mode == "frame":
        f = np.arange(T) // L
        allowed = f[:, None] == f[None, :]
    elif mode == "sga":
        s = sga
        keep = _grid_keep_mask(N, L, gh, gw, s["stride_h"], s["stride_w"],
                               s["phase_h"], s["phase_w"])
        allowed = np.broadcast_to(keep[None, :], (T, T)).copy()
        if s["diagonal"]:
            allowed[np.arange(T), np.arange(T)] = True   # no-op for kept tokens
        nd = int((~keep).sum())
        if s["mean_fill"] and nd > 0:
            kmean = k[~keep].mean(axis=0)                  # [H, d]
            vmean = v[~keep].mean(axis=0)
            zm = scale * np.einsum("ihe,he->hi", q, kmean)  # [H, T]
            if s["mean_fill"] == 2:
                extra_logits = zm[:, :, None]
                vals.append(vmean[:, None, :])
            elif mean_copies:
                extra_logits = np.repeat(zm[:, :, None], nd, axis=2)
                vals.append(np.repeat(vmean[:, None, :], nd, axis=1))
            else:
                extra_logits = (zm + np.log(nd))[:, :, None]
                vals.append(vmean[:, None, :])
    elif mode == "register":
        f = np.arange(T) // L
        special = (np.arange(T) % L) >= gh * gw
        same_frame = f[:, None] == f[None, :]
        both_special = special[:, None] & special[None, :]
        allowed = np.where(special[:, None], both_special, same_frame)
    elif mode != "global":
        raise ValueError(mode)
    z = np.where(allowed[None], z, -np.inf)
    if extra_logits is not None:
        z = np.concatenate([z, extra_logits], axis=2)
    p = _softmax_rows(z)                                   # [H, T, cols]
    vv = np.concatenate(vals, axis=1)                      # [H, cols, d]
    return np.einsum("hic,hce->ihe", p, vv)


def probabilities(mode, q, k, N, L, gh, gw, scale, sga=None):
    """The row-stochastic matrix [H, T, T(+1)] of the same softmax (for pins)."""
    T, H, d = q.shape
    eye_v = np.zeros((T, H, T))
    # value rows = one-hot over key index: output row == probability row
    for h in range(H):
        eye_v[:, h, :] = np.eye(T)
    vpad = eye_v
    out = attention(mode, q, k, vpad, N, L, gh, gw, scale, sga)
    return out.transpose(1, 0, 2)
