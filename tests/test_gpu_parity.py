"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Pages: "10 · R4 — decode split-attention dim-parallel rewrite" (sections 2.1,
2.2, 3.2, 4: the chunk-boundary parity sweep) and "Red Lite dev35 — long-context
decode: grouped split-K attention" (Change: grouped workgroups, block length).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_records, parity, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

HEAD_DIMS = (8, 16, 32, 64, 128, 256)
GROUPS = (1, 2, 3, 4, 5, 6, 7, 8)


def _ref(case):
    return oracle.decode_attn(case.q, case.k, case.v, case.positions,
                              case.shape.n_kv_head, case.scale)


def _records(case, S, blk=0):
    return oracle.split_partials(case.q, case.k, case.v, case.positions,
                                 case.shape.n_kv_head, case.scale, S, blk)


def test_tiny_config_records_and_output():
    """1 layer, 4q/2kv, hd 64, nkv 256, 4 splits."""
    case = synth.make_case(1, synth.CFG1, 256, poison_tail=True)
    say("tiny cfg", "S=4")
    out, rec = run_gpu(case, synth.CFG1_SPLITS)
    parity(out, _ref(case), "tiny out", "1 tiny 4q/2kv hd64")
    check_records(rec, _records(case, synth.CFG1_SPLITS), "tiny records",
                  "1 tiny 4q/2kv hd64")


@pytest.mark.parametrize("hd", HEAD_DIMS)
def test_every_instantiation(hd):
    """Every compiled (head_dim, group) pair on ragged lengths and splits."""
    for G in GROUPS:
        nkvh = 2
        shape = synth.Shape(2, nkvh * G, nkvh, hd, 320)
        case = synth.make_case(100 + G, shape, [300, 77], poison_tail=True)
        ref = _ref(case)
        dev = to_device(case)
        for S in (1, 3, 7):
            say(f"hd={hd} G={G} S={S}")
            out, rec = run_gpu(case, S, dev=dev)
            parity(out, ref, f"hd={hd} G={G} S={S}", "instantiations (hd, G)")
            check_records(rec, _records(case, S), f"hd={hd} G={G} S={S}",
                          "instantiations (hd, G)")


def test_chunk_boundary_sweep():
    """Live lengths at multiples of the chunk and their neighbours (idle splits)."""
    shape = synth.Shape(1, 28, 4, 128, 2100)
    S = 32
    base = synth.make_case(2, shape, shape.max_ctx)
    dev = to_device(base)
    lengths = sorted({1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129, 1023,
                      1024, 1025, 2047, 2048, 2049, 2100} |
                     {m * c + d for c in (4, 16, 64) for m in (1, 5, 31)
                      for d in (-1, 0, 1)})
    for nkv in lengths:
        base.positions[:] = nkv - 1
        dev[3].fill_(nkv - 1)
        say(f"boundary nkv={nkv}")
        out, rec = run_gpu(base, S, dev=dev)
        parity(out, _ref(base), f"nkv={nkv}", "chunk-boundary sweep 28q/4kv")
        lo, hi = oracle.split_bounds(nkv, S)
        lohi = rec[0, :, 0, 2:4].copy().view(np.int32)
        assert np.array_equal(lohi[:, 0], lo) and np.array_equal(lohi[:, 1], hi)


def test_empty_and_single_row():
    """nkv = 0 gives exact zeros; nkv = 1 gives V[0] bit for bit."""
    shape = synth.Shape(3, 8, 2, 128, 64)
    case = synth.make_case(3, shape, [1, 0, 64], poison_tail=True)
    case.positions[:] = [0, -1, 10**9]          # 1 row, empty, clamped to 64
    for S, blk in ((1, 0), (4, 0), (64, 0), (2, 32)):
        say(f"edges S={S} blk={blk}")
        out, rec = run_gpu(case, S, blk)
        G = shape.group
        for h in range(shape.n_head):
            assert np.array_equal(out[0, h], case.v[0, 0, h // G].astype(np.float32))
            assert np.array_equal(out[1, h], np.zeros(shape.head_dim, np.float32))
        parity(out, _ref(case), f"edges S={S}", "edges nkv 0/1/clamped")
        check_records(rec, _records(case, S, blk), f"edges S={S} blk={blk}",
                      "edges nkv 0/1/clamped")


@pytest.mark.parametrize("hd", [16, 128])
def test_int32_extreme_positions(hd):
    """positions at the int32 extremes: INT32_MAX is clamped to max_ctx
    (no overflow of positions + 1), INT32_MIN is an empty context."""
    shape = synth.Shape(3, 8, 2, hd, 64)
    case = synth.make_case(9, shape, [64, 0, 6], poison_tail=True)
    case.positions[:] = [2**31 - 1, -2**31, 5]
    for S, blk in ((1, 0), (5, 0), (64, 0), (2, 32)):
        say(f"int32 extreme positions hd={hd} S={S} blk={blk}")
        out, rec = run_gpu(case, S, blk)
        assert np.array_equal(out[1], np.zeros_like(out[1]))
        parity(out, _ref(case), f"int32 positions hd={hd} S={S}",
               "edges nkv 0/1/clamped")
        check_records(rec, _records(case, S, blk), f"int32 positions S={S}",
                      "edges nkv 0/1/clamped")


def test_7b_2k_split_sweep():
    """28q/4kv hd 128 at nkv 2048 over the swept split counts."""
    case = synth.make_case(2, synth.CFG2, 2048)
    ref = _ref(case)
    dev = to_device(case)
    for S in synth.CFG2_SPLIT_SWEEP:
        say(f"7b@2k S={S}")
        out, rec = run_gpu(case, S, dev=dev)
        parity(out, ref, f"7b@2k S={S}", "2 7B 28q/4kv hd128 nkv 2048")
        check_records(rec, _records(case, S), f"7b@2k S={S}",
                      "2 7B 28q/4kv hd128 nkv 2048")


def test_hd256_block_lengths():
    """16q/2kv hd 256 at nkv 8400 with fixed block lengths 32..256."""
    case = synth.make_case(4, synth.CFG4, synth.CFG4_NKV)
    ref = _ref(case)
    dev = to_device(case)
    for blk in synth.CFG4_BLOCKS:
        S = -(-synth.CFG4.max_ctx // blk)
        say(f"hd256 blk={blk} S={S}")
        out, rec = run_gpu(case, S, blk, dev=dev)
        parity(out, ref, f"hd256 blk={blk}", "4 hd256 16q/2kv nkv 8400")
        check_records(rec, _records(case, S, blk), f"hd256 blk={blk}",
                      "4 hd256 16q/2kv nkv 8400")


def test_growing_context_offsets():
    """Score offsets up to +-20 per 128 rows, lengths 2^k-1 .. 2^k+1, k=7..15."""
    import decode_attention_gqa_amd as skv
    sh = synth.CFG3
    case = synth.make_offset_case(3, sh, sh.max_ctx)
    dev = to_device(case)
    S_h, blk_h = skv.pick_splits(sh.batch, sh.n_head, sh.n_kv_head, sh.head_dim,
                                 sh.max_ctx, 256)
    for nkv in synth.CFG3_LENGTHS:
        case.positions[:] = nkv - 1
        dev[3].fill_(nkv - 1)
        ref = _ref(case)
        for S, blk in ((S_h, blk_h), (64, 0), (258, 128)):
            say(f"growing nkv={nkv} S={S} blk={blk}")
            out, _ = run_gpu(case, S, blk, dev=dev)
            parity(out, ref, f"growing nkv={nkv} S={S} blk={blk}",
                   "3 growing 28q/4kv hd128 +-20 offsets")


def _oracle_per_sequence(case):
    """The oracle one sequence at a time on a thread pool (the C oracle runs
    with the GIL released); the same values as one call over the batch."""
    import concurrent.futures as cf
    import os
    B = case.shape.batch

    def one(b):
        return oracle.decode_attn(case.q[b:b + 1], case.k[b:b + 1],
                                  case.v[b:b + 1], case.positions[b:b + 1],
                                  case.shape.n_kv_head, case.scale)
    with cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        return np.concatenate(list(ex.map(one, range(B))))


def test_ragged_batch_full():
    """32 sequences, 32q/8kv hd 128, nkv_b ~ U{512..32768}: the full-size
    launch at the heuristic's split count, every output of all 32 sequences
    against the oracle, and every sequence's split bounds bit-exact."""
    import decode_attention_gqa_amd as skv
    sh = synth.CFG5
    lengths = synth.cfg5_lengths()
    case = synth.make_case(5, sh, lengths, poison_tail=True)
    S, blk = skv.pick_splits(sh.batch, sh.n_head, sh.n_kv_head, sh.head_dim,
                             sh.max_ctx, 256)
    say(f"ragged B=32 S={S}")
    out, rec = run_gpu(case, S, blk)
    say("ragged oracle, 32 sequences")
    parity(out, _oracle_per_sequence(case), "ragged batch",
           "5 ragged 32x 32q/8kv hd128")
    for b in range(sh.batch):
        lo, hi = oracle.split_bounds(int(lengths[b]), S, blk)
        lohi = rec[b, :, 0, 2:4].copy().view(np.int32)
        assert np.array_equal(lohi[:, 0], lo) and np.array_equal(lohi[:, 1], hi)


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_large_magnitude_q(hd):
    """Queries far from N(0, 1), on the matrix-core path (q enters as fp16 hi
    + lo pairs of q * scale * log2(e), which must stay below 65504).

    q x 30: the scores of a group spread over about +-130 natural-log units,
    so the online softmax's reference max jumps often and the query parts sit
    at high fp16 exponents; outputs and every split record are held to the
    bar.
    q x 4000: every head's softmax is one-hot (output = its top row's V) and
    the query's hi parts reach ~2^11. Outputs are held to the bar; of the
    records only the structure (bounds, idle pattern, finite values) is
    checked: scores of ~10^4 base-2 units carry ~1e-3 units of rounding in any
    fp32 evaluation, so a split whose two best rows lie within a few units of
    each other has records that move by up to ~1e-3 (its output weight is
    then negligible against the head's best row)."""
    import decode_attention_gqa_amd as skv
    G = 8 if hd == 256 else 7
    nkvh = 2 if hd == 256 else 4
    shape = synth.Shape(1, nkvh * G, nkvh, hd, 8400)
    base = synth.make_case(7, shape, 8400, poison_tail=True)
    S_h, _ = skv.pick_splits(1, shape.n_head, nkvh, hd, shape.max_ctx, 256)
    for factor in (30.0, 4000.0):
        q = (base.q * np.float32(factor)).astype(np.float32)
        qmax = float(np.abs(q).max()) * base.scale * 1.4426950408889634
        assert qmax < 65504.0, qmax
        case = synth.Case(shape, q, base.k, base.v, base.positions.copy(),
                          base.scale)
        dev = to_device(case)
        full = factor < 100
        label = ("large q x30 (outputs and records)" if full
                 else "large q x4000 (outputs)")
        for nkv in (8400, 3001):
            case.positions[:] = nkv - 1
            dev[3].fill_(nkv - 1)
            ref = _ref(case)
            for S in (S_h, 7):
                say(f"large q hd={hd} x{factor} nkv={nkv} S={S}")
                out, rec = run_gpu(case, S, dev=dev)
                parity(out, ref, f"large q hd={hd} x{factor} nkv={nkv} S={S}",
                       label)
                want = _records(case, S)
                if full:
                    check_records(rec, want, f"large q hd={hd} x{factor} S={S}",
                                  label)
                else:
                    lohi = rec[..., 2:4].copy().view(np.int32)
                    assert np.array_equal(lohi, want[..., 2:4].astype(np.int32))
                    idle = want[..., 0] == -np.inf
                    assert np.array_equal(rec[..., 0] == -np.inf, idle)
                    assert np.all(np.isfinite(rec[..., 1:][~idle]))


@pytest.mark.parametrize("hd", [8, 16])
def test_precision_stress(hd):
    """hd 8 / 16, 4q/2kv, nkv 1024: fp32 q keeps the bar."""
    sh = synth.CFG5P[hd]
    case = synth.make_case(6, sh, synth.CFG5P_NKV)
    ref = _ref(case)
    dev = to_device(case)
    for S in (1, 4, 16, 64):
        say(f"precision hd={hd} S={S}")
        out, rec = run_gpu(case, S, dev=dev)
        parity(out, ref, f"precision hd={hd} S={S}", f"5p precision hd{hd}")
        check_records(rec, _records(case, S), f"precision hd={hd} S={S}",
                      f"5p precision hd{hd}")


def test_deterministic():
    case = synth.make_case(2, synth.CFG2, 1500)
    dev = to_device(case)
    say("determinism")
    a, _ = run_gpu(case, 32, dev=dev)
    b, _ = run_gpu(case, 32, dev=dev)
    assert np.array_equal(a, b)
