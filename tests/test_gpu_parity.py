"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars (from the arithmetic the kernels use):
* fp32 inputs: max-abs error <= 1e-5;
* bf16 inputs (fp32 accumulation, bf16 P and O): max-abs <= 1.5e-2 and
  mean-abs <= 2e-3, against the oracle run on the same bf16 bits;
* SGA keep_idx / keep_mask: bit-exact; kmean / vmean (fp32 sums): within
  1e-5 of the mean absolute dropped value, in absolute terms.
Small cases compare every output; the full-size workloads (100, 300 and 800
frames of 37x37+5 tokens, 16 heads, and the largest shape the ABI accepts,
1,526 frames) compare seeded sampled rows, which the oracle computes one by
one.  The same bars apply to register attention, the
unit-weight mean column and the row-range calls (whose rows are also
compared with the same rows of the full call).  Twenty seeded random small
configurations (grid, specials, heads, SGA strides, phases and flags) add
breadth in both element types.
"""
import math
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
        if mode == "register":
            out = vga.register_attn(q, k, v, frames)[0]
        else:
            fn = vga.frame_attn if mode == "frame" else vga.global_attn
            out = fn(q, k, v, frames)
        torch.cuda.synchronize()
        code = {"frame": oracle.MODE_FRAME, "global": oracle.MODE_GLOBAL,
                "register": oracle.MODE_REGISTER}[mode]
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
    run_and_compare(vga, frames, q, k, v, ["frame", "global", "register"],
                    [vga.Sga(2, 2, 0, 0, True, True), vga.Sga(2, 2, 0, 0, False, True),
                     vga.Sga(2, 2, 0, 0, True, False), vga.Sga(3, 3, 1, 1, True, True),
                     vga.Sga(2, 2, 0, 0, True, 2)],
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
    (2, 8, 8, 0, 1),      # L = 64: exactly one key tile, no ragged tile
    (2, 4, 8, 0, 2),      # L = 32: one ragged tile whose second half is empty
    (1, 8, 12, 0, 1),     # L = 96: a ragged 32-key tile plus one full tile
    (3, 5, 13, 0, 1),     # L = 65: a one-key ragged tile plus one full tile
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
        sgas.append(vga.Sga(2, 2, 1, 1, True, 2))     # unit-weight mean column
    sgas.append(vga.Sga(1, 1, 0, 0, True, True))      # nothing dropped: no mean column
    run_and_compare(vga, frames, q, k, v, ["frame", "global", "register"], sgas,
                    tag="%s-%s" % (shape, dt))


@pytest.mark.parametrize("nb_last", range(1, 17))
def test_ragged_workgroup_blocks(vga, nb_last):
    # One frame of L = 507 + 32 * nb_last tokens: the second 512-query
    # workgroup holds nb_last 32-row blocks, the last of them 27 rows.  The
    # bf16 kernel spreads them over its waves (one, two or no blocks each)
    # and skips absent blocks; every output row is compared.
    L = 507 + 32 * nb_last
    frames = vga.Frames(1, 2, (L - 1) // 2, 1, 2)
    assert frames.tokens == L
    q, k, v = to_dev(tiny_qkv(L, 2, 64, seed=300 + nb_last), torch.bfloat16)
    run_and_compare(vga, frames, q, k, v, ["frame", "global"],
                    [vga.Sga(2, 2, 0, 0, True, True)], tag="nb_last=%d" % nb_last)


@pytest.mark.parametrize("dt,H", [("bf16", 64), ("f32", 32)])
def test_most_heads(vga, dt, H):
    # the largest head counts the ABI accepts (64 in bf16, 32 in fp32): the
    # gather then moves the widest rows, 1,024 chunks of 16 bytes per token
    frames = vga.Frames(3, 6, 7, 2, H)
    q, k, v = to_dev(tiny_qkv(frames.tokens, H, 64, seed=77),
                     torch.float32 if dt == "f32" else torch.bfloat16)
    run_and_compare(vga, frames, q, k, v, ["frame", "global", "register"],
                    [vga.Sga(2, 2, 0, 0, True, True), vga.Sga(3, 2, 1, 1, True, 2)],
                    tag="H=%d-%s" % (H, dt))
    with pytest.raises(vga.VgaError) as ei:
        more = vga.Frames(3, 6, 7, 2, H + 1)
        x = torch.zeros(more.tokens, H + 1, 64, device="cuda", dtype=q.dtype)
        vga.global_attn(x, x, x, more)
    assert ei.value.status == 8


def test_sga_flag_combinations_bf16(vga):
    frames = vga.Frames(3, 9, 8, 2, 2)
    q, k, v = to_dev(tiny_qkv(frames.tokens, 2, 64, seed=7), torch.bfloat16)
    run_and_compare(vga, frames, q, k, v, [],
                    [vga.Sga(2, 3, 1, 2, d, mfill) for d in (False, True) for mfill in (0, 1, 2)],
                    tag="flags")


def planted_jump_qkv(frames, jump_log2, seed):
    """Q, K, V whose every query scores two planted keys about `jump_log2`
    (log2 units) above the rest: q = b*u + noise, k = a*u at tokens 198 (a
    kept patch of frame 1: the last full global tile, a full frame tile,
    compacted index 38+ under SGA 2x2) and 290 (a special token of frame 1:
    the second 32-key sub-tile of the global tail tile, which runs first);
    other keys are small.  Scale 1/8: logit = a*b/8 nats."""
    rng = np.random.default_rng(seed)
    T, H = frames.tokens, frames.num_heads
    u = rng.standard_normal(64)
    u /= np.linalg.norm(u)
    ab = jump_log2 * 8.0 / math.log2(math.e)
    a = b = math.sqrt(ab)
    q = b * u[None, None, :] + 0.5 * rng.standard_normal((T, H, 64))
    k = 0.5 * rng.standard_normal((T, H, 64))
    v = rng.standard_normal((T, H, 64))
    for t in (198, 290):
        k[t] = a * u[None, :]
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


@pytest.mark.parametrize("jump", [24, 180])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_reference_max_jumps(vga, jump, dt):
    # The bf16 kernel fixes its reference max m at the exact max of the
    # first 32-key sub-tile it processes (the ragged tail tile runs first)
    # and uses P = exp2(S - m) afterwards.  A jump of 24 log2 units keeps
    # every P finite (up to 2^24): the main loop's result must stand.  A
    # jump of 180 overflows P to inf in the main loop, so only the exact
    # fallback loop (taken when a row sum or output is not finite) can give
    # the oracle's answer: passing this case shows that loop ran and is
    # right, for global, frame and SGA attention alike.
    frames = vga.Frames(2, 12, 12, 2, 2)       # L = 146, T = 292: tail tiles everywhere
    assert frames.tokens == 292
    q, k, v = to_dev(planted_jump_qkv(frames, jump, seed=jump), dt)
    run_and_compare(vga, frames, q, k, v, ["frame", "global"], [vga.Sga(2, 2, 0, 0)],
                    tag="jump%d" % jump)


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


def test_graph_replay(vga):
    # the calls enqueue kernels only (no memset, no allocation, no host sync),
    # so they can be captured in a graph: every replay, with eager work and
    # synchronisation between replays, equals the eager result bit for bit
    frames = vga.Frames(3, 9, 8, 2, 2)
    q, k, v = to_dev(tiny_qkv(frames.tokens, 2, 64, seed=21), torch.bfloat16)
    sga = vga.Sga(2, 2, 0, 0)
    ref = {"global": vga.global_attn(q, k, v, frames).clone()}
    o, ws = vga.sga_attn(q, k, v, frames, sga)
    ref["sga"] = o.clone()
    o, rws = vga.register_attn(q, k, v, frames)
    ref["register"] = o.clone()
    outs = {m: torch.empty_like(q) for m in ref}

    def calls():
        vga.global_attn(q, k, v, frames, out=outs["global"])
        vga.sga_attn(q, k, v, frames, sga, out=outs["sga"], workspace=ws)
        vga.register_attn(q, k, v, frames, out=outs["register"], workspace=rws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for i in range(4):
        for t in outs.values():
            t.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for m in ref:
            assert torch.equal(outs[m], ref[m]), (i, m)


def test_concurrent_streams(vga):
    # two problems in flight on two streams give the results they give alone
    fa = vga.Frames(4, 10, 10, 3, 2)
    fb = vga.Frames(2, 7, 9, 5, 3)
    qa, ka, va = to_dev(tiny_qkv(fa.tokens, 2, 64, seed=31), torch.bfloat16)
    qb, kb, vb = to_dev(tiny_qkv(fb.tokens, 3, 64, seed=32), torch.bfloat16)
    sga = vga.Sga(2, 3, 1, 0)
    alone_a = vga.global_attn(qa, ka, va, fa).clone()
    alone_b = vga.sga_attn(qb, kb, vb, fb, sga)[0].clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a, outs_b = [], []
    for _ in range(3):
        with torch.cuda.stream(s1):
            outs_a.append(vga.global_attn(qa, ka, va, fa))
        with torch.cuda.stream(s2):
            outs_b.append(vga.sga_attn(qb, kb, vb, fb, sga)[0])
    torch.cuda.synchronize()
    for a, b in zip(outs_a, outs_b):
        assert torch.equal(a, alone_a) and torch.equal(b, alone_b)


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
    with pytest.raises(ValueError):
        vga.sga_select(q, q.float(), frames, vga.Sga())
    with pytest.raises(ValueError):
        vga.sga_select(q[:8], q[:8], frames, vga.Sga())


# --------------------------------------------- projections around a layer
# Bars for y = x W^T + b (fp32 accumulation over K = 64 H terms).  fp32
# path (one sequential FMA chain of K + 1 terms per output): the
# probabilistic bound of Higham and Mary ("A new approach to probabilistic
# rounding error analysis", SIAM J. Sci. Comput. 41(5), 2019, theorem 2.4),
# |err| <= 1e-5 + lam sqrt(K + 1) 2^-24 (sum_k |x_k w_k| + |b|) with lam = 8,
# which holds with probability at least 1 - 2 (K + 1) exp(-lam^2 / 2)
# (5e-11 per element at K = 2048) when the rounding errors are independent;
# the sum of magnitudes comes from the oracle on |x|, |w|, |b|.  The
# worst-case bound (K + 1) 2^-24 (...) is sqrt(K + 1) / 8 times looser (up to
# 5.7x here).  bf16 path: |err| <= 2^-8 |y| + 2^-10 per element -- the RNE
# rounding of y to bf16 (at most 2^-9 |y|) plus the fp32 accumulation.
PROJ_SHAPES = [
    # N, gh, gw, S, H -- ragged token counts; C = 128..1024; 3C not a
    # multiple of the 256-wide feature tile for H = 2, 3
    (3, 7, 9, 3, 2),
    (5, 11, 13, 4, 3),
    (2, 16, 16, 1, 4),
    (1, 20, 20, 5, 16),
]


def check_linear(got, ref, dtype, what, absdot=None, K=None):
    err = np.abs(as_f64(got) - ref)
    say("  %s: max-abs %.3g (|y| max %.3g)" % (what, float(err.max()), float(np.abs(ref).max())))
    if dtype == "f32":
        assert absdot is not None and K is not None, what
        assert np.all(err <= F32_MAX + 8.0 * math.sqrt(K + 1) * 2.0 ** -24 * absdot), what
    else:
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -10), what


@pytest.mark.parametrize("shape", PROJ_SHAPES, ids=lambda s: "N%d_%dx%d_S%d_H%d" % s)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_projections(vga, shape, dt):
    N, gh, gw, S, H = shape
    frames = vga.Frames(N, gh, gw, S, H)
    T, C = frames.tokens, 64 * H
    rng = np.random.default_rng(500 + 7 * H + N)
    x = rng.standard_normal((T, C)).astype(np.float32)
    w = (rng.standard_normal((3 * C, C)) / math.sqrt(C)).astype(np.float32)
    b = rng.standard_normal(3 * C).astype(np.float32)
    wo = (rng.standard_normal((C, C)) / math.sqrt(C)).astype(np.float32)
    bo = rng.standard_normal(C).astype(np.float32)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    xd, wd, bd, wod, bod = to_dev((x, w, b, wo, bo), tdt)
    for bias in (True, False):
        say("case proj-%s %s bias=%s" % (dt, shape, bias))
        q, k, v = vga.qkv_proj(xd, wd, bd if bias else None, frames)
        torch.cuda.synchronize()
        rq, rk, rv = oracle.qkv_proj(host(xd), host(wd), host(bd) if bias else None, H)
        aq, ak, av = (None,) * 3
        if dt == "f32":
            aq, ak, av = oracle.qkv_proj(np.abs(host(xd)), np.abs(host(wd)),
                                         np.abs(host(bd)) if bias else None, H)
        for name, got, ref, ab in (("q", q, rq, aq), ("k", k, rk, ak), ("v", v, rv, av)):
            check_linear(host(got), ref, dt, "qkv %s" % name, ab, C)
        y = vga.out_proj(q, wod, bod if bias else None, frames)
        torch.cuda.synchronize()
        ry = oracle.linear(host(q).reshape(T, C), host(wod), host(bod) if bias else None)
        ay = None
        if dt == "f32":
            ay = oracle.linear(np.abs(host(q).reshape(T, C)), np.abs(host(wod)),
                               np.abs(host(bod)) if bias else None)
        check_linear(host(y), ry, dt, "out", ay, C)


def test_projection_bias_element_aligned_bf16(vga):
    # the ABI asks the bias to be aligned to its element only: a bf16 bias
    # starting 2 bytes past a 16-byte boundary gives the same result as an
    # aligned copy of it (and the oracle's)
    frames = vga.Frames(3, 7, 9, 3, 2)
    T, C = frames.tokens, 128
    rng = np.random.default_rng(811)
    x = rng.standard_normal((T, C)).astype(np.float32)
    w = (rng.standard_normal((3 * C, C)) / math.sqrt(C)).astype(np.float32)
    b = rng.standard_normal(3 * C + 1).astype(np.float32)
    xd, wd, bfull = to_dev((x, w, b), torch.bfloat16)
    bshift = bfull[1:]                        # data_ptr 2 bytes past the allocation
    assert bshift.data_ptr() % 16 == 2 and bshift.is_contiguous()
    baligned = bshift.clone()
    say("case proj-bias-offset bf16")
    got = vga.qkv_proj(xd, wd, bshift, frames)
    ref_gpu = vga.qkv_proj(xd, wd, baligned, frames)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj(host(xd), host(wd), host(baligned), 2)
    for g, r, ro in zip(got, ref_gpu, (rq, rk, rv)):
        assert torch.equal(g, r)
        check_linear(host(g), ro, "bf16", "qkv, bias at +2 bytes")


@pytest.mark.parametrize("dt,H", [("bf16", 64), ("f32", 32)])
def test_projections_most_heads(vga, dt, H):
    # the widest rows the ABI accepts: C = 4096 (bf16, W_qkv 12,288 x 4,096)
    # and C = 2048 (fp32); 45 tokens, a ragged token tile
    frames = vga.Frames(3, 3, 4, 3, H)
    T, C = frames.tokens, 64 * H
    rng = np.random.default_rng(640 + H)
    x = rng.standard_normal((T, C)).astype(np.float32)
    w = (rng.standard_normal((3 * C, C)) / math.sqrt(C)).astype(np.float32)
    b = rng.standard_normal(3 * C).astype(np.float32)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    xd, wd, bd = to_dev((x, w, b), tdt)
    say("case proj-most-heads %s H=%d" % (dt, H))
    q, k, v = vga.qkv_proj(xd, wd, bd, frames)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj(host(xd), host(wd), host(bd), H)
    aq, ak, av = (None,) * 3
    if dt == "f32":
        aq, ak, av = oracle.qkv_proj(np.abs(host(xd)), np.abs(host(wd)), np.abs(host(bd)), H)
    for name, got, ref, ab in (("q", q, rq, aq), ("k", k, rk, ak), ("v", v, rv, av)):
        check_linear(host(got), ref, dt, "qkv %s" % name, ab, C)
    wo = wd[:C].contiguous()
    y = vga.out_proj(q, wo, None, frames)
    torch.cuda.synchronize()
    ay = None
    if dt == "f32":
        ay = oracle.linear(np.abs(host(q).reshape(T, C)), np.abs(host(wo)))
    check_linear(host(y), oracle.linear(host(q).reshape(T, C), host(wo)), dt, "out", ay, C)


# ------------------------------------------- feature-field workloads (sampled)
def _ff(vga, w):
    frames = vga.Frames(w.num_frames, w.grid_h, w.grid_w, w.num_special, w.num_heads)
    q, k, v = vga_inputs.feature_field_qkv(w.num_frames, w.grid_h, w.grid_w, w.num_special,
                                           w.num_heads, 64, seed=w.seed, device="cuda")
    return frames, q, k, v


def _rows_with_tail(T, count, seed, L):
    rows = seeded_rows(T, count, seed)
    # frame edges, query-tile edges, and the first and last special of frames
    extra = np.array([0, 1, L - 1, L, T - 257, T - 256, T - 2, T - 1, L - 5, 2 * L - 5,
                      T // 2 // L * L + L - 3])
    return np.unique(np.concatenate([rows, extra[(extra >= 0) & (extra < T)]]))


def test_n4_worked_example(vga):
    frames, q, k, v = _ff(vga, vga_inputs.N4)
    rows = _rows_with_tail(frames.tokens, 600, 41, frames.tokens_per_frame)
    run_and_compare(vga, frames, q, k, v, ["frame", "global", "register"],
                    [vga.Sga(2, 2, 0, 0), vga.Sga(3, 3, 1, 1), vga.Sga(2, 2, 0, 0, True, 2)],
                    rows=rows, tag="N=4")


def test_n100_full_size(vga):
    frames, q, k, v = _ff(vga, vga_inputs.N100)
    rows = _rows_with_tail(frames.tokens, 96, 42, frames.tokens_per_frame)
    run_and_compare(vga, frames, q, k, v, ["frame", "global", "register"],
                    [vga.Sga(2, 2, 0, 0)], rows=rows, tag="N=100")


def test_n300_full_size_sga(vga):
    frames, q, k, v = _ff(vga, vga_inputs.N300)
    rows = _rows_with_tail(frames.tokens, 48, 43, frames.tokens_per_frame)
    run_and_compare(vga, frames, q, k, v, [], [vga.Sga(2, 2, 0, 0)], rows=rows, tag="N=300")


def test_n800_full_size_frame_sga(vga):
    frames, q, k, v = _ff(vga, vga_inputs.N800)
    rows = _rows_with_tail(frames.tokens, 32, 44, frames.tokens_per_frame)
    run_and_compare(vga, frames, q, k, v, ["frame", "register"], [vga.Sga(3, 3, 1, 1)],
                    rows=rows, tag="N=800")
    # exact global attention over all 1,099,200 keys, on fewer sampled rows
    # (the oracle's cost per row is the whole key set)
    grow = np.unique(np.concatenate([seeded_rows(frames.tokens, 12, 46),
                                     [0, frames.tokens - 1]]))
    run_and_compare(vga, frames, q, k, v, ["global"], [], rows=grow, tag="N=800")


def test_max_size_bf16(vga):
    # the largest shape the ABI accepts at 16 heads: T*H*64 < 2^31 elements
    # per tensor, 1,526 frames of 37x37+5 (T = 2,096,724; 4.3 GB per tensor)
    L, H = 37 * 37 + 5, 16
    N = (2 ** 31 // (H * 64) - 1) // L
    assert N * L * H * 64 < 2 ** 31 <= (N + 1) * L * H * 64
    frames = vga.Frames(N, 37, 37, 5, H)
    q, k, v = vga_inputs.feature_field_qkv(N, 37, 37, 5, H, 64, seed=6, device="cuda")
    T = frames.tokens
    rows = _rows_with_tail(T, 16, 47, L)
    run_and_compare(vga, frames, q, k, v, ["frame", "register"], [vga.Sga(3, 3, 1, 1)],
                    rows=rows, tag="max")
    # exact global attention for the last 700 query rows against all T keys
    r0 = T - 700
    say("case max global rows [%d, %d)" % (r0, T))
    out = vga.global_attn_rows(q[r0:].contiguous(), k, v, frames, r0)
    torch.cuda.synchronize()
    sel = np.unique(np.concatenate([seeded_rows(700, 6, 48) + r0, [r0, T - 1]]))
    ref = oracle.attention(oracle.MODE_GLOBAL, host(q), host(k), host(v), N, L, 37, 37, 0.125,
                           rows=sel)
    check(host(out[torch.from_numpy(sel - r0).cuda()]), ref, "bf16", "max global rows")


def test_projections_max_size_bf16(vga):
    # the largest token count the ABI accepts at 16 heads (1,526 frames,
    # T = 2,096,724): x is 4,294,090,752 bytes, so the kernel's 32-bit DMA
    # offsets into x come within 876 KB of 2^32; sampled rows incl. the last
    L, H = 37 * 37 + 5, 16
    N = (2 ** 31 // (H * 64) - 1) // L
    frames = vga.Frames(N, 37, 37, 5, H)
    T, C = frames.tokens, 64 * H
    assert T * C * 2 < 2 ** 32 < (T + 512) * C * 2
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    x = torch.randn(T, C, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(3 * C, C, device="cuda", generator=g) / 32).to(torch.bfloat16)
    b = torch.randn(3 * C, device="cuda", generator=g).to(torch.bfloat16)
    say("case proj-max T=%d" % T)
    q, k, v = vga.qkv_proj(x, w, b, frames)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([seeded_rows(T, 24, 50), [0, T - 257, T - 256, T - 1]]))
    sel = torch.from_numpy(rows).cuda()
    rq, rk, rv = oracle.qkv_proj(host(x[sel]), host(w), host(b), H)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_linear(host(got[sel]), ref, "bf16", "max qkv %s" % name)
    del k, v
    y = vga.out_proj(q, w[:C].contiguous(), None, frames)
    torch.cuda.synchronize()
    ry = oracle.linear(host(q[sel]).reshape(len(rows), C), host(w[:C].contiguous()))
    check_linear(host(y[sel]), ry, "bf16", "max out")


# ------------------------------------------------------------ row-range calls
def _range_cases(T, L):
    # empty, one row, unaligned, tile-straddling, whole frames, everything
    return [(0, 0), (5, 6), (3, min(T, 70)), (max(0, T - 300), T - 1), (L, min(T, 3 * L)),
            (0, T)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rows_small(vga, dt):
    frames = vga.Frames(5, 11, 13, 4, 2)          # L = 147, T = 735
    T, L = frames.tokens, frames.tokens_per_frame
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    q, k, v = to_dev(tiny_qkv(T, 2, 64, seed=123), tdt)
    qh, kh, vh = host(q), host(k), host(v)
    sga = vga.Sga(2, 3, 1, 0, True, 1)
    full = {"global": vga.global_attn(q, k, v, frames),
            "frame": vga.frame_attn(q, k, v, frames),
            "sga": vga.sga_attn(q, k, v, frames, sga)[0]}
    for r0, r1 in _range_cases(T, L):
        rows = np.arange(r0, r1)
        for mode in ("global", "frame", "sga"):
            if mode == "frame" and (r0 % L or r1 % L):
                with pytest.raises(vga.VgaError) as ei:
                    vga.frame_attn_rows(q[r0:r1].contiguous(), k, v, frames, r0)
                assert ei.value.status == 2
                continue
            say("case rows-%s %s [%d, %d)" % (dt, mode, r0, r1))
            qr = q[r0:r1].contiguous()
            if mode == "global":
                out = vga.global_attn_rows(qr, k, v, frames, r0)
            elif mode == "frame":
                out = vga.frame_attn_rows(qr, k, v, frames, r0)
            else:
                out = vga.sga_attn_rows(qr, k, v, frames, sga, r0)[0]
            torch.cuda.synchronize()
            assert out.shape[0] == r1 - r0
            if r1 == r0:
                continue
            code = {"global": oracle.MODE_GLOBAL, "frame": oracle.MODE_FRAME,
                    "sga": oracle.MODE_SGA}[mode]
            ref = oracle.attention(code, qh, kh, vh, frames.num_frames, L, 11, 13, 0.125,
                                   oracle_sga(sga) if mode == "sga" else None, rows=rows)
            check(host(out), ref, dt, "rows %s [%d,%d)" % (mode, r0, r1))
            # the same rows of the full call: identical in fp32 (one lane per
            # query); in bf16 a shard may take the exact-max path on other tiles
            a, b = out.float(), full[mode][r0:r1].float()
            if dt == "f32":
                assert torch.equal(a, b), mode
            else:
                assert float((a - b).abs().max()) <= BF16_MAX


def test_rows_n100_one_of_eight(vga):
    # one device's share when 100 frames are split over 8 devices by query
    # rows: rows [3T/8, 4T/8) against all 137,400 keys
    frames, q, k, v = _ff(vga, vga_inputs.N100)
    T, L = frames.tokens, frames.tokens_per_frame
    r0, r1 = 3 * T // 8, 4 * T // 8
    qh, kh, vh = host(q), host(k), host(v)
    rows = np.unique(np.concatenate([seeded_rows(r1 - r0, 48, 45) + r0,
                                     [r0, r0 + 1, r1 - 2, r1 - 1]]))
    say("case rows-N100 global [%d, %d)" % (r0, r1))
    out = vga.global_attn_rows(q[r0:r1].contiguous(), k, v, frames, r0)
    torch.cuda.synchronize()
    ref = oracle.attention(oracle.MODE_GLOBAL, qh, kh, vh, 100, L, 37, 37, 0.125, rows=rows)
    check(host(out[torch.from_numpy(rows - r0).cuda()]), ref, "bf16", "N=100 rows global")
    sga = vga.Sga(2, 2, 0, 0)
    say("case rows-N100 sga [%d, %d)" % (r0, r1))
    out = vga.sga_attn_rows(q[r0:r1].contiguous(), k, v, frames, sga, r0)[0]
    torch.cuda.synchronize()
    ref = oracle.attention(oracle.MODE_SGA, qh, kh, vh, 100, L, 37, 37, 0.125, oracle_sga(sga),
                           rows=rows)
    check(host(out[torch.from_numpy(rows - r0).cuda()]), ref, "bf16", "N=100 rows sga")


def test_block_n100_full_size(vga):
    # a whole global block at 100 frames, as the block benchmark runs it: the
    # QKV projection (137,400 x 1024 -> 3 x 1024, a ragged last token tile),
    # exact global attention and the output projection, on sampled rows
    N, gh, gw, S, H = 100, 37, 37, 5, 16
    frames = vga.Frames(N, gh, gw, S, H)
    T, L, C = frames.tokens, frames.tokens_per_frame, 64 * H
    x, w, b, wo, bo = vga_inputs.feature_field_block(N, gh, gw, S, H, seed=12, device="cuda")
    rows = _rows_with_tail(T, 48, 49, L)
    sel = torch.from_numpy(rows).cuda()
    say("case block-N100 qkv_proj T=%d" % T)
    q, k, v = vga.qkv_proj(x, w, b, frames)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj(host(x[sel]), host(w), host(b), H)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_linear(host(got[sel]), ref, "bf16", "block qkv %s" % name)
    say("case block-N100 global")
    o = vga.global_attn(q, k, v, frames)
    torch.cuda.synchronize()
    ref = oracle.attention(oracle.MODE_GLOBAL, host(q), host(k), host(v), N, L, gh, gw, 0.125,
                           rows=rows)
    check(host(o[sel]), ref, "bf16", "block global")
    say("case block-N100 out_proj")
    y = vga.out_proj(o, wo, bo, frames)
    torch.cuda.synchronize()
    assert y.shape == (T, C)
    ry = oracle.linear(host(o[sel]).reshape(len(rows), C), host(wo), host(bo))
    check_linear(host(y[sel]), ry, "bf16", "block out")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_sga_select_matches_attn(vga, dt):
    # the selection call alone leaves the same workspace (bit for bit) as the
    # attention call: same kernels, fixed-order sums; checked against the
    # oracle's selection and mean too
    frames = vga.Frames(3, 7, 9, 3, 2)
    T = frames.tokens
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    q, k, v = to_dev(tiny_qkv(T, 2, 64, seed=77), tdt)
    code = vga.VGA_F32 if dt == "f32" else vga.VGA_BF16
    for p in (vga.Sga(2, 2, 0, 0), vga.Sga(3, 2, 1, 1, False, 2)):
        say("case select-%s %s" % (dt, p))
        _, ws_a = vga.sga_attn(q, k, v, frames, p)
        ws_b = vga.sga_select(k, v, frames, p)
        torch.cuda.synchronize()
        a, b = vga.workspace_views(ws_a, frames, p, code), vga.workspace_views(ws_b, frames, p, code)
        for name in ("keep_idx", "keep_mask", "kmean", "vmean", "kc", "vc"):
            assert torch.equal(a[name], b[name]), name
        r = resolved(p, vga)
        idx, mask = oracle.select(3, frames.tokens_per_frame, 7, 9, r.stride_h, r.stride_w,
                                  r.phase_h, r.phase_w)
        assert np.array_equal(b["keep_idx"].cpu().numpy().astype(np.int64), idx)
        km, vm, nd = oracle.dropped_mean(host(k), host(v), 3, frames.tokens_per_frame, 7, 9,
                                         r.stride_h, r.stride_w, r.phase_h, r.phase_w)
        assert nd > 0
        assert np.max(np.abs(b["kmean"].cpu().numpy() - km)) <= 1e-5
        assert np.max(np.abs(b["vmean"].cpu().numpy() - vm)) <= 1e-5


@pytest.mark.parametrize("seed", range(20))
def test_random_configurations(vga, seed):
    # seeded random small configurations: frame count, grid, specials, heads,
    # SGA strides, phases and flags, in both element types, every output
    rng = np.random.default_rng(900 + seed)
    N = int(rng.integers(1, 5))
    gh, gw = int(rng.integers(1, 12)), int(rng.integers(1, 12))
    S = int(rng.integers(0, 6))
    H = int(rng.integers(1, 4))
    dt = "f32" if seed % 2 == 0 else "bf16"
    frames = vga.Frames(N, gh, gw, S, H)
    q, k, v = to_dev(tiny_qkv(frames.tokens, H, 64, seed=1000 + seed),
                     torch.float32 if dt == "f32" else torch.bfloat16)
    sgas = []
    for _ in range(3):
        sh, sw = int(rng.integers(1, gh + 1)), int(rng.integers(1, gw + 1))
        sgas.append(vga.Sga(sh, sw, int(rng.integers(-1, sh)), int(rng.integers(-1, sw)),
                            bool(rng.integers(0, 2)), int(rng.integers(0, 3))))
    run_and_compare(vga, frames, q, k, v, ["frame", "global", "register"], sgas,
                    tag="random%d-%s N%d %dx%d S%d H%d" % (seed, dt, N, gh, gw, S, H))
