"""GPU: the KV-cache append kernel (dotLLM issue #199, comment 1, section 1,
the cache update that a decode step performs ahead of attention).

The caches after an append must equal the oracle's bit for bit (NaN
patterns compare as NaN), for every head size, rows per call and position
mix, including positions whose rows fall partly or wholly outside the cache.
A captured graph of one decode step (append + partial + combine) replayed
with positions[] advancing must match the oracle's step-by-step result.
"""
import numpy as np
import pytest

import oracle
from gpu_util import parity, say, torch_mod

pytestmark = pytest.mark.gpu

I32_MAX, I32_MIN = 2**31 - 1, -2**31


def _f16_equal(got, ref, what):
    got = np.asarray(got).view(np.uint16)
    ref = np.asarray(ref).view(np.uint16)
    nan_g = ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
    nan_r = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x3FF) != 0)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions differ"
    bad = np.flatnonzero((got != ref) & ~nan_r)
    assert bad.size == 0, (f"{what}: {bad.size} fp16 patterns differ, first "
                           f"flat index {bad[0]}")


def _new_rows(rng, B, n, nkvh, hd):
    x = (rng.standard_normal((B, n, nkvh, hd)) * 30).astype(np.float32)
    # values that test the rounding: ties, overflow, subnormals, specials
    special = np.array([np.nan, np.inf, -np.inf, 65504.0, 65519.996, 65520.0,
                        -7e4, 2.0**-24, 2.0**-25, 3 * 2.0**-26, 1e-30, -0.0,
                        1.0 + 2.0**-11, 1.0 + 3 * 2.0**-11, 2049.0, 2051.0],
                       np.float32)
    flat = x.reshape(-1)
    m = min(flat.size, special.size)
    flat[:m] = special[:m]
    return x


@pytest.mark.parametrize("hd", [8, 64, 128, 256])
@pytest.mark.parametrize("nkvh", [1, 4, 8])
def test_append_bit_exact(hd, nkvh):
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    rng = np.random.default_rng(hd * 10 + nkvh)
    T = 40
    for n_rows in (1, 3, 7):
        B = 8
        pos = np.array([n_rows - 1, 17, T - 1, T + 2, 1, -5, I32_MAX, I32_MIN],
                       np.int32)
        kc = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
        vc = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
        kn = _new_rows(rng, B, n_rows, nkvh, hd)
        vn = _new_rows(rng, B, n_rows, nkvh, hd)[:, :, ::-1].copy()
        want_k, want_v = oracle.append_kv(kn, vn, kc, vc, pos)
        d = [torch.from_numpy(a).cuda() for a in (kn, vn, kc, vc, pos)]
        say(f"append hd={hd} nkvh={nkvh} n_rows={n_rows}")
        skv.append_kv(*d)
        torch.cuda.synchronize()
        _f16_equal(d[2].cpu().numpy(), want_k, f"K hd={hd} n={n_rows}")
        _f16_equal(d[3].cpu().numpy(), want_v, f"V hd={hd} n={n_rows}")


def test_decode_step_graph():
    """One graph = append the new row, then attention over the grown cache.
    Replayed for 12 steps with positions[] and the new rows updated between
    replays (outside the graph); each step's output matches the oracle run
    on the oracle's own appended cache, and the final caches are equal bit
    for bit."""
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    rng = np.random.default_rng(7)
    B, nh, nkvh, hd, T = 2, 28, 4, 128, 512
    scale = float(np.float32(1 / np.sqrt(hd)))
    k = np.zeros((B, T, nkvh, hd), np.float16)
    v = np.zeros((B, T, nkvh, hd), np.float16)
    start = np.array([100, 255], np.int32)       # rows before these exist
    k[:, :300] = rng.standard_normal((B, 300, nkvh, hd)).astype(np.float16)
    v[:, :300] = rng.standard_normal((B, 300, nkvh, hd)).astype(np.float16)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    S, blk = skv.pick_splits(B, nh, nkvh, hd, T, cu)
    dk, dv = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    q_d = torch.empty((B, nh, hd), device="cuda")
    kn_d = torch.empty((B, 1, nkvh, hd), device="cuda")
    vn_d = torch.empty((B, 1, nkvh, hd), device="cuda")
    pos_d = torch.from_numpy(start.copy()).cuda()
    part = torch.empty(skv.partials_bytes(B, nh, hd, S) // 4, device="cuda")
    out = torch.empty((B, nh, hd), device="cuda")

    def step():
        skv.append_kv(kn_d, vn_d, dk, dv, pos_d)
        skv.decode_attn(q_d, dk, dv, pos_d, part, out, S, blk, scale)

    ck, cv = k.copy(), v.copy()
    graph = None
    for i in range(12):
        pos = start + i
        q = rng.standard_normal((B, nh, hd)).astype(np.float32)
        kn = rng.standard_normal((B, 1, nkvh, hd)).astype(np.float32)
        vn = rng.standard_normal((B, 1, nkvh, hd)).astype(np.float32)
        q_d.copy_(torch.from_numpy(q))
        kn_d.copy_(torch.from_numpy(kn))
        vn_d.copy_(torch.from_numpy(vn))
        pos_d.copy_(torch.from_numpy(pos))
        if graph is None:
            # first step eagerly (also the warm-up), then capture the same step
            say("decode step eager, step 0")
            step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            say(f"decode step capture S={S}")
            # capture records the launches only; nothing runs until replay
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
        else:
            say(f"decode step replay {i}")
            graph.replay()
            torch.cuda.synchronize()
        ck, cv = oracle.append_kv(kn, vn, ck, cv, pos)
        want = oracle.decode_attn(q, ck, cv, pos, nkvh, scale)
        parity(out.cpu().numpy(), want, f"decode step {i}",
               "append + attention graph")
    _f16_equal(dk.cpu().numpy(), ck, "K after 12 steps")
    _f16_equal(dv.cpu().numpy(), cv, "V after 12 steps")
