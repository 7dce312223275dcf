"""Whole plans on the GPU: the per-layer schedules of the training-free
pipeline ("AVGGT: Rethinking Global Attention for Accelerating VGGT",
section 3: early global layers converted to frame attention, the remaining
ones run as SGA), every slot run through ``attention()`` exactly as a trunk
would dispatch it, each output compared with the oracle in that slot's mode;
and one ordinary call with the library's debug synchronisation switched on.

Bars as in test_gpu_parity: bf16 max-abs <= 1.5e-2 and mean-abs <= 2e-3
against the oracle on the same bf16 bits.
"""
import json
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle
from vga_inputs import tiny_qkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BF16_MAX, BF16_MEAN = 1.5e-2, 2e-3


@pytest.fixture(scope="module")
def vga():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import alternating_attention_amd as vga
    return vga


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_out(vga, mode, p, qh, kh, vh, frames, cache):
    key = (mode, p)
    if key not in cache:
        code = {vga.MODE_FRAME: oracle.MODE_FRAME, vga.MODE_GLOBAL: oracle.MODE_GLOBAL,
                vga.MODE_SGA: oracle.MODE_SGA, vga.MODE_REGISTER: oracle.MODE_REGISTER}[mode]
        sga = None
        if mode == vga.MODE_SGA:
            ph = (p.stride_h - 1) // 2 if p.phase_h == -1 else p.phase_h
            pw = (p.stride_w - 1) // 2 if p.phase_w == -1 else p.phase_w
            sga = dict(stride_h=p.stride_h, stride_w=p.stride_w, phase_h=ph, phase_w=pw,
                       diagonal=int(p.diagonal), mean_fill=int(p.mean_fill))
        cache[key] = oracle.attention(code, qh, kh, vh, frames.num_frames,
                                      frames.tokens_per_frame, frames.grid_h, frames.grid_w,
                                      0.125, sga)
    return cache[key]


def test_schedule_plans_through_attention(vga):
    frames = vga.Frames(3, 9, 8, 2, 2)     # L = 74, T = 222: ragged tiles
    q, k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16).contiguous()
               for a in tiny_qkv(frames.tokens, 2, 64, seed=77))
    qh, kh, vh = bits(q), bits(k), bits(v)
    plans = {
        "avggt 24 slots": vga.layer_schedule(24, 8, vga.Sga(3, 3, 1, 1)),
        "avggt 3x3": vga.layer_schedule(6, 2, vga.Sga(3, 3, -1, -1)),
        "frame + exact": vga.layer_schedule(5, 2, None),
        "per-slot strides": vga.layer_schedule_sga(
            6, 2, [vga.Sga(2, 2, 0, 0), vga.Sga(3, 3, -1, -1),
                   vga.Sga(2, 3, 1, 0, False, 2), vga.Sga(3, 2, 2, 1, True, 0)]),
        "register every 2nd": vga.layer_schedule_register(7, 2, 2, vga.Sga(2, 2, 0, 0)),
    }
    cache = {}
    seen = set()
    for name, plan in plans.items():
        for slot, (mode, p) in enumerate(plan):
            say("plan %s slot %d mode %d %s" % (name, slot, mode, p))
            out = vga.attention(mode, q, k, v, frames, p)
            torch.cuda.synchronize()
            ref = oracle_out(vga, mode, p, qh, kh, vh, frames, cache)
            err = np.abs(oracle.bf16_bits_to_f64(bits(out)) - ref)
            assert float(err.max()) <= BF16_MAX and float(err.mean()) <= BF16_MEAN, \
                (name, slot, float(err.max()), float(err.mean()))
            seen.add(mode)
    assert seen == {vga.MODE_FRAME, vga.MODE_GLOBAL, vga.MODE_SGA, vga.MODE_REGISTER}


DEBUG_CHILD = r"""
import json, sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import alternating_attention_amd as vga
from vga_inputs import tiny_qkv
frames = vga.Frames(4, 37, 37, 5, 2)     # T = 5,496: long enough to still run if not synced
q, k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16).contiguous()
           for a in tiny_qkv(frames.tokens, 2, 64, seed=5))
torch.cuda.synchronize()
res = {}
o = vga.global_attn(q, k, v, frames)
res["idle_after_global"] = torch.cuda.current_stream().query()
s, ws = vga.sga_attn(q, k, v, frames, vga.Sga(2, 2, 0, 0))
res["idle_after_sga"] = torch.cuda.current_stream().query()
r, rws = vga.register_attn(q, k, v, frames)
res["idle_after_register"] = torch.cuda.current_stream().query()
res["last_error"] = vga.last_error()
np.save(sys.argv[2] + "_global.npy", o.view(torch.int16).cpu().numpy())
np.save(sys.argv[2] + "_sga.npy", s.view(torch.int16).cpu().numpy())
np.save(sys.argv[2] + "_register.npy", r.view(torch.int16).cpu().numpy())
print(json.dumps(res))
"""


def test_debug_sync_call(vga):
    # VGA_DEBUG_SYNC=1 (read once per process) makes every call wait for its
    # kernels and report execution errors as VGA_ERR_HIP.  In a child
    # process with it set, ordinary calls succeed, the stream is idle as each
    # call returns, and the outputs equal those of this process bit for bit.
    frames = vga.Frames(4, 37, 37, 5, 2)
    q, k, v = (torch.from_numpy(a).cuda().to(torch.bfloat16).contiguous()
               for a in tiny_qkv(frames.tokens, 2, 64, seed=5))
    ref = {"global": vga.global_attn(q, k, v, frames),
           "sga": vga.sga_attn(q, k, v, frames, vga.Sga(2, 2, 0, 0))[0],
           "register": vga.register_attn(q, k, v, frames)[0]}
    torch.cuda.synchronize()
    with tempfile.TemporaryDirectory() as td:
        base = os.path.join(td, "out")
        env = dict(os.environ, VGA_DEBUG_SYNC="1")
        say("case debug-sync child process")
        r = subprocess.run([sys.executable, "-c", DEBUG_CHILD, ROOT, base], env=env,
                           capture_output=True, text=True, timeout=240)
        assert r.returncode == 0, r.stderr[-2000:]
        res = json.loads(r.stdout.strip().splitlines()[-1])
        assert res["idle_after_global"] and res["idle_after_sga"] and res["idle_after_register"]
        assert res["last_error"] == ""
        for name, t in ref.items():
            got = np.load(base + "_%s.npy" % name)
            assert np.array_equal(got, t.view(torch.int16).cpu().numpy()), name
