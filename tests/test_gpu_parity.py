"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars (from the arithmetic the kernels use):
* fp32 inputs: max-abs error <= 1e-5;
* bf16 inputs (fp32 accumulation, bf16 P and O): max-abs <= 1.5e-2 and
  mean-abs <= 2e-3, against the oracle run on the same bf16 bits;
* SGA keep_idx / keep_mask: bit-exact; kmean / vmean (fp32 sums): within
  1e-5 of the mean absolute dropped value, in absolute terms.
Small cases compare every output; the full-size workloads (100, 300 and 800
frames of 37x37+5 tokens, 16 heads) compare seeded sampled rows, which the
oracle computes one by one.
"""
import sys

import numpy as np
import pytest

import oracle
import vga_inputs
from vga_inputs import seeded_rows, tiny_qkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32_MAX = 1e-5
BF16_MAX, BF16_MEAN = 1.5e-2, 2e-3


@pytest.fixture(scope="module")
def vga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import alternating_attention_amd as vga
    return vga


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def host(t):
    """GPU tensor -> numpy (fp32 as is, bf16 as raw uint16 bits)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a):
    return oracle.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def check(got, ref, dtype, what):
    err = np.abs(as_f64(got) - ref)
    mx, mean = float(err.max()), float(err.mean())
    say("  %s: max-abs %.3g mean-abs %.3g" % (what, mx, mean))
    if dtype == "f32":
        assert mx <= F32_MAX, what
    else:
        assert mx <= BF16_MAX and mean <= BF16_MEAN, what


def oracle_sga(p: "vga.Sga"):
    return dict(stride_h=p.stride_h, stride_w=p.stride_w, phase_h=p.phase_h,
                phase_w=p.phase_w, diagonal=int(p.diagonal), mean_fill=int(p.mean_fill))


def resolved(p, vga):
    ph = (p.stride_h - 1) // 2 if p.phase_h == -1 else p.phase_h
    pw = (p.stride_w - 1) // 2 if p.phase_w == -1 else p.phase_w
    return vga.Sga(p.stride_h, p.stride_w, ph, pw, p.diagonal, p.mean_fill)


def run_and_compare(vga, frames, q, k, v, modes, sga_list=(), rows=None, tag=""):
    """Run each mode on the GPU and compare to the oracle on `rows` (None: all)."""
    dtype = "f32" if q.dtype == torch.float32 else "bf16"
    qh, kh, vh = host(q), host(k), host(v)
    N, L, gh, gw = frames.num_frames, frames.tokens_per_frame, frames.grid_h, frames.grid_w
    scale = 1.0 / 8.0
    sel = slice(None) if rows is None else torch.from_numpy(rows).to(q.device)
    for mode in modes:
        say("case %s mode=%s T=%d H=%d" % (tag, mode, frames.tokens, frames.num_heads))
        fn = vga.frame_attn if mode == "frame" else vga.global_attn
        out = fn(q, k, v, frames)
        torch.cuda.synchronize()
        code = oracle.MODE_FRAME if mode == "frame" else oracle.MODE_GLOBAL
        ref = oracle.attention(code, qh, kh, vh, N, L, gh, gw, scale, rows=rows)
        check(host(out[sel]), ref, dtype, "%s %s" % (tag, mode))
    for p in sga_list:
        p = resolved(p, vga)
        say("case %s mode=sga %s T=%d" % (tag, p, frames.tokens))
        out, ws = vga.sga_attn(q, k, v, frames, p)
        torch.cuda.synchronize()
        views = vga.workspace_views(ws, frames, p,
                                    vga.VGA_F32 if dtype == "f32" else vga.VGA_BF16)
        idx, mask = oracle.select(N, L, gh, gw, p.stride_h, p.stride_w, p.phase_h, p.phase_w)
        assert np.array_equal(views["keep_idx"].cpu().numpy().astype(np.int64), idx)
        assert np.array_equal(views["keep_mask"].cpu().numpy(), mask)
        # compacted rows are exact copies
        kc = host(views["kc"])
        assert np.array_equal(kc, kh[idx]), "Kc is not K[keep_idx]"
        assert np.array_equal(host(views["vc"]), vh[idx]), "Vc is not V[keep_idx]"
        km, vm, nd = oracle.dropped_mean(kh, vh, N, L, gh, gw, p.stride_h, p.stride_w,
                                         p.phase_h, p.phase_w)
        if nd > 0:
            drop = mask == 0
            kscale = float(np.abs(as_f64(kh[drop])).mean())
            vscale = float(np.abs(as_f64(vh[drop])).mean())
            assert np.max(np.abs(views["kmean"].cpu().numpy() - km)) <= 1e-5 * kscale
            assert np.max(np.abs(views["vmean"].cpu().numpy() - vm)) <= 1e-5 * vscale
        ref = oracle.attention(oracle.MODE_SGA, qh, kh, vh, N, L, gh, gw, scale,
                               oracle_sga(p), rows=rows)
        check(host(out[sel]), ref, dtype, "%s sga %dx%d" % (tag, p.stride_h, p.stride_w))


def to_dev(arrs, dtype):
    return [torch.from_numpy(a).to("cuda").to(dtype).contiguous() for a in arrs]


# ------------------------------------------------------------ tiny fp32 (full)
def test_tiny_fp32_all_modes(vga):
    w = vga_inputs.TINY
    frames = vga.Frames(w.num_frames, w.grid_h, w.grid_w, w.num_special, w.num_heads)
    q, k, v = to_dev(tiny_qkv(frames.tokens, w.num_heads, 64, w.seed), torch.float32)
    run_and_compare(vga, frames, q, k, v, ["frame", "global"],
                    [vga.Sga(2, 2, 0, 0, True, True), vga.Sga(2, 2, 0, 0, False, True),
                     vga.Sga(2, 2, 0, 0, True, False), vga.Sga(3, 3, 1, 1, True, True)],
                    tag="tiny-f32")


# ---------------------------------------------- small ragged shapes (full)
SHAPES = [
    # N, gh, gw, S, H  -- tile-unaligned L and T, one frame, tiny frames
    (3, 7, 9, 3, 3),
    (1, 5, 5, 0, 1),
    (2, 1, 1, 0, 2),      # L = 1: one token per frame
    (5, 11, 13, 4, 2),    # L = 147 spans several 64-key tiles, T = 735 several q tiles
    (1, 16, 16, 0, 1),    # L = 256: exactly one query tile
    (2, 16, 16, 1, 1),    # L = 257: one row past a tile
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "N%d_%dx%d_S%d_H%d" % s)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_small_shapes(vga, shape, dt):
    N, gh, gw, S, H = shape
    frames = vga.Frames(N, gh, gw, S, H)
    q, k, v = to_dev(tiny_qkv(frames.tokens, H, 64, seed=100 + N * 7 + gh),
                     torch.float32 if dt == "f32" else torch.bfloat16)
    sgas = []
    if gh >= 2 and gw >= 2:
        sgas = [vga.Sga(2, 2, 0, 0, True, True), vga.Sga(min(3, gh), min(2, gw), -1, -1, True, True),
                vga.Sga(gh, gw, 0, 0, True, True)]    # one patch kept per frame
    sgas.append(vga.Sga(1, 1, 0, 0, True, True))      # nothing dropped: no mean column
    run_and_compare(vga, frames, q, k, v, ["frame", "global"], sgas, tag="%s-%s" % (shape, dt))


def test_sga_flag_combinations_bf16(vga):
    frames = vga.Frames(3, 9, 8, 2, 2)
    q, k, v = to_dev(tiny_qkv(frames.tokens, 2, 64, seed=7), torch.bfloat16)
    run_and_compare(vga, frames, q, k, v, [],
                    [vga.Sga(2, 3, 1, 2, d, mfill) for d in (False, True) for mfill in (False, True)],
                    tag="flags")


def test_large_logits_rescale_bf16(vga):
    # peaked rows (|logit| up to ~40) exercise the lazy max update
    frames = vga.Frames(2, 12, 12, 2, 2)
    q, k, v = tiny_qkv(frames.tokens, 2, 64, seed=9)
    q = q * 6.0
    k = k.copy()
    k[frames.tokens // 2:] *= 2.0   # later keys score higher: the max grows mid-row
    q, k, v = to_dev((q, k, v), torch.bfloat16)
    run_and_compare(vga, frames, q, k, v, ["frame", "global"], [vga.Sga(2, 2, 0, 0)],
                    tag="peaked")


def test_deterministic(vga):
    frames = vga.Frames(4, 10, 10, 3, 2)
    q, k, v = to_dev(tiny_qkv(frames.tokens, 2, 64, seed=3), torch.bfloat16)
    a = vga.global_attn(q, k, v, frames).clone()
    b = vga.global_attn(q, k, v, frames)
    assert torch.equal(a, b)
    sa, wa = vga.sga_attn(q, k, v, frames, vga.Sga())
    sa = sa.clone()
    wa = wa.clone()
    sb, wb = vga.sga_attn(q, k, v, frames, vga.Sga())
    assert torch.equal(sa, sb)
    va, vb = vga.workspace_views(wa, frames, vga.Sga()), vga.workspace_views(wb, frames, vga.Sga())
    assert torch.equal(va["kmean"], vb["kmean"]) and torch.equal(va["vmean"], vb["vmean"])


def test_python_errors(vga):
    frames = vga.Frames(1, 4, 4, 0, 1)
    q = torch.zeros(16, 1, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        vga.global_attn(q, q, q.float(), frames)
    with pytest.raises(ValueError):
        vga.global_attn(q[:8], q[:8], q[:8], frames)
    with pytest.raises(vga.VgaError) as ei:
        vga.global_attn(q, q, q, frames, out=q)       # o aliases q
    assert ei.value.status == 6


# ------------------------------------------- feature-field workloads (sampled)
def _ff(vga, w):
    frames = vga.Frames(w.num_frames, w.grid_h, w.grid_w, w.num_special, w.num_heads)
    q, k, v = vga_inputs.feature_field_qkv(w.num_frames, w.grid_h, w.grid_w, w.num_special,
                                           w.num_heads, 64, seed=w.seed, device="cuda")
    return frames, q, k, v


def _rows_with_tail(T, count, seed, L):
    rows = seeded_rows(T, count, seed)
    extra = np.array([0, 1, L - 1, L, T - 257, T - 256, T - 2, T - 1])
    return np.unique(np.concatenate([rows, extra[(extra >= 0) & (extra < T)]]))


def test_n4_worked_example(vga):
    frames, q, k, v = _ff(vga, vga_inputs.N4)
    rows = _rows_with_tail(frames.tokens, 600, 41, frames.tokens_per_frame)
    run_and_compare(vga, frames, q, k, v, ["frame", "global"],
                    [vga.Sga(2, 2, 0, 0), vga.Sga(3, 3, 1, 1)], rows=rows, tag="N=4")


def test_n100_full_size(vga):
    frames, q, k, v = _ff(vga, vga_inputs.N100)
    rows = _rows_with_tail(frames.tokens, 96, 42, frames.tokens_per_frame)
    run_and_compare(vga, frames, q, k, v, ["frame", "global"], [vga.Sga(2, 2, 0, 0)],
                    rows=rows, tag="N=100")


def test_n300_full_size_sga(vga):
    frames, q, k, v = _ff(vga, vga_inputs.N300)
    rows = _rows_with_tail(frames.tokens, 48, 43, frames.tokens_per_frame)
    run_and_compare(vga, frames, q, k, v, [], [vga.Sga(2, 2, 0, 0)], rows=rows, tag="N=300")


def test_n800_full_size_frame_sga(vga):
    frames, q, k, v = _ff(vga, vga_inputs.N800)
    rows = _rows_with_tail(frames.tokens, 32, 44, frames.tokens_per_frame)
    run_and_compare(vga, frames, q, k, v, ["frame"], [vga.Sga(3, 3, 1, 1)], rows=rows,
                    tag="N=800")
