"""Beam-decode attention over a shared context KV on the GPU against the fp64
oracle (oracle.beam; Semantic-ID GR inference: a shared request-level
ContextKV, short per-beam BeamKV, beam paths -- news.bpdata.com Hungarian
article, section "SID-GR inference").  Tolerances: fp32 rel L2 <= 1e-4;
bf16 rel L2 <= 1e-2 and max abs <= 3e-2 (inputs rounded to bf16 first, so
both sides see the same values)."""
import numpy as np
import pytest
import torch

from gpu_util import tol_check
from hstu_jagged_silu_fwd_amd import beam as hb
from oracle.beam import beam_decode_attention
from workloads import round_bf16

pytestmark = pytest.mark.gpu


def make(seed, R, W, Hq, Hkv, d, ctx, Cmax, S, dtype):
    rng = np.random.default_rng(seed)
    rnd = (lambda a: round_bf16(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32).astype(np.float64))
    q = rnd(rng.normal(0, 1, size=(R, W, Hq, d)))
    ck = rnd(rng.normal(0, 1, size=(R, Hkv, Cmax, d)))
    cv = rnd(rng.normal(0, 1, size=(R, Hkv, Cmax, d)))
    bk = rnd(rng.normal(0, 1, size=(R, S, W, Hkv, d)))
    bv = rnd(rng.normal(0, 1, size=(R, S, W, Hkv, d)))
    return dict(q=q, ck=ck, cv=cv, bk=bk, bv=bv, ctx=np.array(ctx, np.int32), rng=rng)


def run(c, path, t, dtype, scale, out_fill=None):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda a, dt=tdt: torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dt)
    q = dev(c["q"])
    out = torch.full_like(q, 5.0 if out_fill is None else out_fill)
    ws = hb.decode_attn(q, dev(c["ck"]), dev(np.swapaxes(c["cv"], 2, 3)), dev(c["ctx"], torch.int32),
                        dev(c["bk"]), dev(c["bv"]), None if t == 0 else dev(path, torch.int32), out, t, scale)
    torch.cuda.synchronize()
    return out, int(ws[:4].view(torch.int32).item())


def oracle(c, path, t, scale):
    ctx_k = [np.swapaxes(c["ck"][r, :, :n], 0, 1) for r, n in enumerate(c["ctx"])]
    ctx_v = [np.swapaxes(c["cv"][r, :, :n], 0, 1) for r, n in enumerate(c["ctx"])]
    return beam_decode_attention(c["q"], ctx_k, ctx_v, c["bk"], c["bv"], path, t, scale)


CASES = [
    # (dtype, d, R, W, Hq, Hkv, ctx, Cmax, t)
    ("f32", 128, 3, 40, 4, 2, [0, 37, 300], 320, 2),
    ("f32", 64, 2, 7, 6, 3, [96, 1], 128, 0),
    ("bf16", 128, 3, 40, 4, 2, [0, 37, 300], 320, 2),
    ("bf16", 64, 2, 130, 2, 1, [513, 64], 544, 1),
    ("bf16", 128, 2, 256, 16, 8, [1000, 517], 1024, 2),
    ("f32", 64, 1, 1, 2, 2, [40], 64, 3),          # one beam, no grouping, a 4-token path
    ("bf16", 128, 3, 3, 8, 2, [63, 64, 65], 96, 1),  # lengths around a 64-key step
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-W{c[3]}-t{c[8]}" for c in CASES])
def test_beam_decode_matches_oracle(case):
    dtype, d, R, W, Hq, Hkv, ctx, Cmax, t = case
    print(f"case beam {case}", flush=True)
    c = make(11, R, W, Hq, Hkv, d, ctx, Cmax, t + 1, dtype)
    path = c["rng"].integers(0, W, size=(R, W, t)).astype(np.int32)
    scale = d ** -0.5
    out, code = run(c, path, t, dtype, scale)
    assert code == 0, f"device status {code}"
    tol_check(out.float().cpu().numpy(), oracle(c, path, t, scale), dtype, f"beam {case}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_loop_with_beam_selection(dtype):
    """Three decode steps: each step writes its tokens' K/V into BeamKV slot
    (t, w), then new beams pick parents; a new beam's path is its parent's
    path followed by the parent's slot.  Every step is checked."""
    print(f"case beam decode loop {dtype}", flush=True)
    R, W, Hq, Hkv, d, Cmax, S = 2, 24, 4, 2, 128, 256, 3
    c = make(12, R, W, Hq, Hkv, d, [200, 33], Cmax, S, dtype)
    rng = c["rng"]
    rnd = (lambda a: round_bf16(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32).astype(np.float64))
    path = np.zeros((R, W, 0), np.int32)
    for t in range(S):
        c["q"] = rnd(rng.normal(0, 1, size=(R, W, Hq, d)))
        out, code = run(c, path, t, dtype, d ** -0.5)
        assert code == 0
        tol_check(out.float().cpu().numpy(), oracle(c, path, t, d ** -0.5), dtype, f"loop step {t}")
        parent = rng.integers(0, W, size=(R, W))
        path = np.concatenate([np.take_along_axis(path, parent[:, :, None].repeat(t, 2), 1) if t else path,
                               parent[:, :, None]], axis=2).astype(np.int32)


def test_device_errors_leave_output_untouched():
    print("case beam errors", flush=True)
    R, W, Hq, Hkv, d, Cmax = 2, 8, 2, 1, 64, 64
    c = make(13, R, W, Hq, Hkv, d, [10, 64], Cmax, 2, "f32")
    path = np.zeros((R, W, 1), np.int32)
    c["ctx"] = np.array([10, 65], np.int32)
    out, code = run(c, path, 1, "f32", 0.125)
    assert code == 9 and torch.all(out == 5.0)
    c["ctx"] = np.array([10, 64], np.int32)
    bad = path.copy()
    bad[1, 3, 0] = W
    out, code = run(c, bad, 1, "f32", 0.125)
    assert code == 10 and torch.all(out == 5.0)
    out, code = run(c, path, 1, "f32", 0.125)
    assert code == 0 and not torch.all(out == 5.0)


def test_beam_decode_at_the_online_size_sampled_beams():
    """Context 5,000, beam 256, 16/8 heads of 128, bf16, step 2: every beam
    computed on the GPU, 6 sampled beams per request against the oracle (the
    oracle needs only their queries and paths; the BeamKV holds all slots)."""
    print("case beam full size sampled", flush=True)
    R, W, Hq, Hkv, d, Cmax, t = 2, 256, 16, 8, 128, 5024, 2
    c = make(14, R, W, Hq, Hkv, d, [5000, 4321], Cmax, t + 1, "bf16")
    path = c["rng"].integers(0, W, size=(R, W, t)).astype(np.int32)
    out, code = run(c, path, t, "bf16", d ** -0.5)
    assert code == 0
    got = out.float().cpu().numpy()
    sel = np.sort(c["rng"].choice(W, size=6, replace=False))
    # the sampled beams' own tokens (step t) move to slots 0..5 of the oracle's
    # copy; earlier steps keep every slot for the paths to index
    bk, bv = c["bk"].copy(), c["bv"].copy()
    bk[:, t, :len(sel)] = c["bk"][:, t, sel]
    bv[:, t, :len(sel)] = c["bv"][:, t, sel]
    sub = dict(c, q=c["q"][:, sel], bk=bk, bv=bv)
    ref = oracle(sub, path[:, sel], t, d ** -0.5)
    tol_check(got[:, sel], ref, "bf16", "beam full size sampled")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scores_that_grow_along_the_context(dtype):
    """Context keys scaled by a ramp over their position, with a large
    softmax scale: the rows' maxima climb by many units of log2 over the
    chunk, by different amounts per row, so the kernel's running reference
    maximum moves on some steps and rows and stays on others (weights up to
    2^8 between moves); the result must not depend on when it moved."""
    print(f"case beam growing scores {dtype}", flush=True)
    R, W, Hq, Hkv, d, Cmax, t = 2, 24, 4, 2, 128, 1024, 1
    c = make(15, R, W, Hq, Hkv, d, [1000, 333], Cmax, t + 1, dtype)
    rnd = (lambda a: round_bf16(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32).astype(np.float64))
    ramp = np.linspace(0.05, 3.0, Cmax)[None, None, :, None]
    c["ck"] = rnd(c["ck"] * ramp)
    path = c["rng"].integers(0, W, size=(R, W, t)).astype(np.int32)
    scale = 0.35
    out, code = run(c, path, t, dtype, scale)
    assert code == 0
    ref = oracle(c, path, t, scale)
    assert np.all(np.isfinite(ref))
    tol_check(out.float().cpu().numpy(), ref, dtype, f"beam growing scores {dtype}")
