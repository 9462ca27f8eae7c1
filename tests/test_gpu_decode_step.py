"""GPU: one decode step with the KV-cache append folded into the partial
kernel (splitkv_decode_step).

dotLLM issue #199, comment 1, section 1 puts the cache update ahead of
attention within a decode step. The folded form
must give, bit for bit, what the append kernel followed by the two-kernel
attention gives (the caches afterwards and the output), and match the fp64
oracle run on the oracle's own appended cache. Positions are chosen so that
the new row falls on the first and the last row of a tile, in every wave's
tiles, in the first and the last split, at row 0, past the cache (nothing is
appended) and before it (no live row).
"""
import numpy as np
import pytest

import oracle
from gpu_util import parity, say, torch_mod

pytestmark = pytest.mark.gpu


def _bits_equal(got, ref, what):
    got = np.ascontiguousarray(got).view(np.uint8)
    ref = np.ascontiguousarray(ref).view(np.uint8)
    assert np.array_equal(got, ref), f"{what}: not bit-identical"


def _run_both(skv, torch, q, kn, vn, k, v, pos, nkvh, S, blk, scale):
    """(out, k, v) of the folded step and of append + attention."""
    dev = [torch.from_numpy(a.copy()).cuda() for a in (k, v, k, v)]
    dq = torch.from_numpy(q).cuda()
    dkn, dvn = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()
    dpos = torch.from_numpy(pos).cuda()
    B, nh, hd = q.shape
    part = [torch.empty(skv.partials_bytes(B, nh, hd, S) // 4, device="cuda")
            for _ in range(2)]
    out = [torch.empty((B, nh, hd), device="cuda") for _ in range(2)]
    skv.decode_step(dq, dkn, dvn, dev[0], dev[1], dpos, part[0], out[0], S,
                    blk, scale)
    skv.append_kv(dkn, dvn, dev[2], dev[3], dpos)
    skv.decode_attn(dq, dev[2], dev[3], dpos, part[1], out[1], S, blk, scale)
    torch.cuda.synchronize()
    return ([o.cpu().numpy() for o in out], [d.cpu().numpy() for d in dev])


@pytest.mark.parametrize("hd,nh,nkvh", [(32, 8, 2), (64, 16, 2), (128, 28, 4),
                                        (128, 8, 8), (256, 16, 2)])
def test_folded_step_equals_separate_calls(hd, nh, nkvh):
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    rng = np.random.default_rng(hd + nh)
    T = 700
    # new-row positions: tile starts and ends, each wave's tiles, row 0, the
    # cache's last row, past the cache (no append), no live row at all
    pos = np.array([0, 15, 16, 63, 64 + 17, 299, 300, 511, T - 1, T + 5, -1],
                   np.int32)
    B = pos.size
    scale = float(np.float32(1 / np.sqrt(hd)))
    k = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
    v = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
    q = rng.standard_normal((B, nh, hd)).astype(np.float32)
    kn = rng.standard_normal((B, 1, nkvh, hd)).astype(np.float32)
    vn = rng.standard_normal((B, 1, nkvh, hd)).astype(np.float32)
    ck, cv = oracle.append_kv(kn, vn, k, v, pos)
    want = oracle.decode_attn(q, ck, cv, pos, nkvh, scale)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    S_h, blk_h = skv.pick_splits(B, nh, nkvh, hd, T, cu)
    for S, blk in ((S_h, blk_h), (1, 0), (7, 0), (12, 64), (44, 16)):
        say(f"decode step hd={hd} nh={nh} nkvh={nkvh} S={S} blk={blk}")
        (o_fold, o_sep), (k_f, v_f, k_s, v_s) = _run_both(
            skv, torch, q, kn, vn, k, v, pos, nkvh, S, blk, scale)
        _bits_equal(k_f, k_s, f"K hd={hd} S={S}")
        _bits_equal(v_f, v_s, f"V hd={hd} S={S}")
        _bits_equal(k_f, ck, f"K vs oracle hd={hd} S={S}")
        _bits_equal(v_f, cv, f"V vs oracle hd={hd} S={S}")
        _bits_equal(o_fold, o_sep, f"out hd={hd} S={S}")
        parity(o_fold, want, f"decode step hd={hd} S={S} blk={blk}",
               "decode step (append folded)")


def test_folded_step_graph():
    """The folded step captured once and replayed for 12 steps with
    positions[] and the new rows updated between replays."""
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    rng = np.random.default_rng(11)
    B, nh, nkvh, hd, T = 2, 28, 4, 128, 512
    scale = float(np.float32(1 / np.sqrt(hd)))
    k = np.zeros((B, T, nkvh, hd), np.float16)
    v = np.zeros((B, T, nkvh, hd), np.float16)
    start = np.array([60, 250], np.int32)
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
        skv.decode_step(q_d, kn_d, vn_d, dk, dv, pos_d, part, out, S, blk,
                        scale)

    ck, cv = k.copy(), v.copy()
    graph = None
    for i in range(12):
        pos = start + 3 * i
        q = rng.standard_normal((B, nh, hd)).astype(np.float32)
        kn = rng.standard_normal((B, 1, nkvh, hd)).astype(np.float32)
        vn = rng.standard_normal((B, 1, nkvh, hd)).astype(np.float32)
        q_d.copy_(torch.from_numpy(q))
        kn_d.copy_(torch.from_numpy(kn))
        vn_d.copy_(torch.from_numpy(vn))
        pos_d.copy_(torch.from_numpy(pos))
        if graph is None:
            say("folded step eager, step 0")
            step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            say(f"folded step capture S={S}")
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
        else:
            say(f"folded step replay {i}")
            graph.replay()
            torch.cuda.synchronize()
        ck, cv = oracle.append_kv(kn, vn, ck, cv, pos)
        want = oracle.decode_attn(q, ck, cv, pos, nkvh, scale)
        parity(out.cpu().numpy(), want, f"folded step {i}",
               "decode step (append folded)")
    _bits_equal(dk.cpu().numpy(), ck, "K after 12 steps")
    _bits_equal(dv.cpu().numpy(), cv, "V after 12 steps")
