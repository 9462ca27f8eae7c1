"""GPU: several query rows per sequence (dotLLM issue #199, comment 1,
section 2: seqQ > 1 with the causal mask starting at positionOffset), the
speculative-verification / chunked-prefill shape, against the oracle's
decode_attn_rows (each row a one-row decode at its own position).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import parity, records_view, say, torch_mod

pytestmark = pytest.mark.gpu


def _rows_case(seed, B, n_q, nh, nkvh, hd, T, pos):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, n_q, nh, hd)).astype(np.float32)
    k = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
    v = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
    return q, k, v, np.asarray(pos, np.int32)


def _run_rows(q, k, v, pos, S, blk, scale):
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    B, n_q, nh, hd = q.shape
    d = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (q, k, v, pos)]
    part = torch.full((skv.partials_bytes(B, n_q * nh, hd, S) // 4,),
                      float("nan"), device="cuda")
    out = torch.full((B, n_q, nh, hd), float("nan"), device="cuda")
    skv.decode_attn_rows(d[0], d[1], d[2], d[3], part, out, S, blk, scale)
    torch.cuda.synchronize()
    rec = records_view(part.cpu().numpy(), B, S, n_q * nh, hd)
    return out.cpu().numpy(), rec


@pytest.mark.parametrize("hd", [8, 16, 32, 64, 128, 256])
def test_rows_parity(hd):
    T = 300
    # rows share a workgroup when their (row, head) pairs fit its columns:
    # G * R <= 8 in one block, G * R <= 16 in two blocks (hd 64 and 128; the
    # last block partly filled when n_q is not a multiple of R)
    for G, nkvh in ((1, 2), (2, 2), (3, 1), (4, 2), (5, 1), (6, 1), (7, 1),
                    (8, 1)):
        nh = G * nkvh
        for n_q in (1, 2, 3, 5, 8):
            # prefill from empty, a chunk mid-cache, at the end, rows before 0
            pos = [n_q - 1, 150, T - 1, 1]
            q, k, v, p = _rows_case(hd + 10 * G + n_q, 4, n_q, nh, nkvh, hd, T, pos)
            scale = float(np.float32(1 / np.sqrt(hd)))
            want = oracle.decode_attn_rows(q, k, v, p, nkvh, scale)
            # split counts that are multiples of 8 launch the blocks of rows
            # of one split side by side (the paired grid)
            for S, blk in ((1, 0), (7, 0), (10, 32), (16, 0), (8, 64)):
                say(f"rows hd={hd} G={G} n_q={n_q} S={S} blk={blk}")
                got, rec = _run_rows(q, k, v, p, S, blk, scale)
                parity(got, want, f"rows hd={hd} G={G} n_q={n_q} S={S}",
                       "rows n_q 1..8, 300 rows")
                # slots [2],[3]: the split bounds of the last row's length
                for b in range(4):
                    lo, hi = oracle.split_bounds(
                        oracle.live_length(int(p[b]), T), S, blk)
                    lohi = rec[b, :, :, 2:4].copy().view(np.int32)
                    assert np.array_equal(lohi[..., 0], np.repeat(
                        lo[:, None], n_q * nh, 1)), (b, S)
                    assert np.array_equal(lohi[..., 1], np.repeat(
                        hi[:, None], n_q * nh, 1)), (b, S)
                # a row before position 0 sees no keys: exactly 0
                if n_q > 2:
                    assert np.all(got[3, 0] == 0.0)


@pytest.mark.parametrize("n_q", [4, 8])
def test_rows_full_length(n_q):
    """The verification shape at the full cache length: 28q/4kv hd 128,
    max_ctx 33,024, two sequences whose last rows sit at 32,767 and 30,000,
    n_q query rows each, at the heuristic's split count (a multiple of 8, so
    the blocks of rows of one split run side by side) and at 64 splits; rows
    past each sequence's end are fp16 NaN so that a read past a row's end
    shows up."""
    import decode_attention_gqa_amd as skv
    B, nh, nkvh, hd, T = 2, 28, 4, 128, 33024
    pos = [32767, 30000]
    q, k, v, p = _rows_case(50 + n_q, B, n_q, nh, nkvh, hd, T, pos)
    for b in range(B):
        k[b, pos[b] + 1:].view(np.uint16)[...] = 0x7E00
        v[b, pos[b] + 1:].view(np.uint16)[...] = 0x7E00
    scale = float(np.float32(1 / np.sqrt(hd)))
    say(f"rows full length n_q={n_q}: oracle")
    want = oracle.decode_attn_rows(q, k, v, p, nkvh, scale)
    S_h, blk_h = skv.pick_splits_rows(B, n_q, nh, nkvh, hd, T, 256)
    assert S_h % 8 == 0, S_h
    for S, blk in ((S_h, blk_h), (64, 0)):
        say(f"rows full length n_q={n_q} S={S}")
        got, rec = _run_rows(q, k, v, p, S, blk, scale)
        parity(got, want, f"rows full length n_q={n_q} S={S}",
               "rows n_q 4/8, 28q/4kv at 32K")
        for b in range(B):
            lo, hi = oracle.split_bounds(pos[b] + 1, S, blk)
            lohi = rec[b, :, 0, 2:4].copy().view(np.int32)
            assert np.array_equal(lohi[:, 0], lo) and \
                np.array_equal(lohi[:, 1], hi)



def test_rows_int32_extreme_positions():
    """Several query rows at positions near the int32 extremes: the rows of
    positions[b] = INT32_MAX all see the whole cache (clamped), those of
    INT32_MIN none (each row's position is computed without overflow)."""
    T, nkvh, n_q = 64, 2, 4
    for G, hd in ((7, 128), (2, 64), (1, 16)):
        nh = G * nkvh
        q, k, v, p = _rows_case(40 + G, 3, n_q, nh, nkvh, hd, T, [T - 1, 0, 5])
        p[:] = [2**31 - 1, -2**31, 5]
        scale = float(np.float32(1 / np.sqrt(hd)))
        want = oracle.decode_attn_rows(q, k, v, p, nkvh, scale)
        for S in (1, 8, 16):
            what = f"rows int32 positions G={G} hd={hd} S={S}"
            say(what)
            got, _ = _run_rows(q, k, v, p, S, 0, scale)
            assert np.array_equal(got[1], np.zeros_like(got[1])), what
            parity(got, want, what, "rows n_q 1..8, 300 rows")


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_rows_nonfinite_v_only_later_rows_see(hd):
    """The newest cache rows are seen by the later query rows of a block
    only (the causal mask of #199 comment 1 section 2). With inf, -inf and
    NaN in such V rows, the earlier query rows must be exactly as if those
    rows were absent: finite and within the bar. The rows that see them must
    be non-finite exactly where the oracle is and within the bar elsewhere
    (an inf reaches the product through the two fp16 parts of p, whose sum
    can be NaN where the definition gives +-inf, so only finiteness is
    compared). Row blocks of one and two MFMA column blocks, and the paired
    grid (16 splits)."""
    T = 300
    cases = [(1, 2, 8), (2, 2, 4), (4, 1, 2), (3, 1, 4), (7, 1, 2)]
    for G, nkvh, n_q in cases:
        nh = G * nkvh
        pos = [T - 1, 150, n_q + 20, 64]
        q, k, v, p = _rows_case(700 + hd + G, 4, n_q, nh, nkvh, hd, T, pos)
        # query row t sits at pos - (n_q - 1 - t): cache row pos - j is seen
        # by the query rows t >= n_q - 1 - j only
        poison = [(0, np.inf), (1, np.nan), (2, -np.inf)]
        for b in range(4):
            for j, val in poison:
                if j < n_q - 1:
                    v[b, pos[b] - j, b % nkvh, (7 * j + b) % hd] = val
        scale = float(np.float32(1 / np.sqrt(hd)))
        want = oracle.decode_attn_rows(q, k, v, p, nkvh, scale)
        assert not np.isfinite(want).all()
        for S in (1, 7, 16):
            what = f"rows non-finite V hd={hd} G={G} n_q={n_q} S={S}"
            say(what)
            got, _ = _run_rows(q, k, v, p, S, 0, scale)
            fin = np.isfinite(want)
            assert np.array_equal(np.isfinite(got), fin), what
            parity(got[fin], want[fin], what, "rows, non-finite V in the newest rows")
            # the first query row of every sequence sees none of them
            assert np.isfinite(got[:, 0]).all(), what


def test_one_row_equals_decode():
    """n_q = 1 through the rows entry point is the one-row decode, bit for
    bit, records included."""
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    sh = synth.Shape(2, 28, 4, 128, 4096)
    case = synth.make_case(9, sh, np.array([4096, 1234]))
    d = [torch.from_numpy(np.ascontiguousarray(a)).cuda()
         for a in (case.q, case.k, case.v, case.positions)]
    S = 16
    p1 = torch.empty(skv.partials_bytes(2, 28, 128, S) // 4, device="cuda")
    p2 = torch.empty_like(p1)
    o1 = torch.empty((2, 28, 128), device="cuda")
    o2 = torch.empty((2, 1, 28, 128), device="cuda")
    say("rows n_q=1 vs decode")
    skv.decode_attn(d[0], d[1], d[2], d[3], p1, o1, S, 0, case.scale)
    skv.decode_attn_rows(d[0].view(2, 1, 28, 128), d[1], d[2], d[3], p2, o2, S,
                         0, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(p1.view(torch.int32), p2.view(torch.int32))
    assert torch.equal(o1, o2.view(2, 28, 128))


def test_speculative_verify_graph():
    """One graph = append n_q new K/V rows at the end of each sequence, then
    attend with the n_q query rows (causal inside them). Replayed as the
    sequences grow by n_q per step; matches the oracle's append + rows on
    every replay, with 28q/4kv hd128 and two sequences of different lengths."""
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    rng = np.random.default_rng(11)
    B, n_q, nh, nkvh, hd, T = 2, 4, 28, 4, 128, 2048
    scale = float(np.float32(1 / np.sqrt(hd)))
    k = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
    v = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
    start = np.array([n_q - 1, 1000], np.int32)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    S, blk = skv.pick_splits(B, nh, nkvh, hd, T, cu)
    dk, dv = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    q_d = torch.empty((B, n_q, nh, hd), device="cuda")
    kn_d = torch.empty((B, n_q, nkvh, hd), device="cuda")
    vn_d = torch.empty((B, n_q, nkvh, hd), device="cuda")
    pos_d = torch.from_numpy(start.copy()).cuda()
    part = torch.empty(skv.partials_bytes(B, n_q * nh, hd, S) // 4, device="cuda")
    out = torch.empty((B, n_q, nh, hd), device="cuda")

    def step():
        skv.append_kv(kn_d, vn_d, dk, dv, pos_d)
        skv.decode_attn_rows(q_d, dk, dv, pos_d, part, out, S, blk, scale)

    ck, cv = k.copy(), v.copy()
    graph = None
    for i in range(8):
        pos = start + n_q * i
        q = rng.standard_normal((B, n_q, nh, hd)).astype(np.float32)
        kn = rng.standard_normal((B, n_q, nkvh, hd)).astype(np.float32)
        vn = rng.standard_normal((B, n_q, nkvh, hd)).astype(np.float32)
        q_d.copy_(torch.from_numpy(q))
        kn_d.copy_(torch.from_numpy(kn))
        vn_d.copy_(torch.from_numpy(vn))
        pos_d.copy_(torch.from_numpy(pos))
        if graph is None:
            say("verify step eager")
            step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            say(f"verify step capture S={S}")
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
        else:
            say(f"verify step replay {i}")
            graph.replay()
            torch.cuda.synchronize()
        ck, cv = oracle.append_kv(kn, vn, ck, cv, pos)
        want = oracle.decode_attn_rows(q, ck, cv, pos, nkvh, scale)
        parity(out.cpu().numpy(), want, f"verify step {i}",
               "rows, verification graph")
