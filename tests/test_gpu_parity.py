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
    parity(out, _ref(case), "tiny out")
    check_records(rec, _records(case, synth.CFG1_SPLITS), "tiny records")


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
            parity(out, ref, f"hd={hd} G={G} S={S}")
            check_records(rec, _records(case, S), f"hd={hd} G={G} S={S}")


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
        parity(out, _ref(base), f"nkv={nkv}")
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
        parity(out, _ref(case), f"edges S={S}")
        check_records(rec, _records(case, S, blk), f"edges S={S} blk={blk}")


def test_7b_2k_split_sweep():
    """28q/4kv hd 128 at nkv 2048 over the swept split counts."""
    case = synth.make_case(2, synth.CFG2, 2048)
    ref = _ref(case)
    dev = to_device(case)
    for S in synth.CFG2_SPLIT_SWEEP:
        say(f"7b@2k S={S}")
        out, rec = run_gpu(case, S, dev=dev)
        parity(out, ref, f"7b@2k S={S}")
        check_records(rec, _records(case, S), f"7b@2k S={S}")


def test_hd256_block_lengths():
    """16q/2kv hd 256 at nkv 8400 with fixed block lengths 32..256."""
    case = synth.make_case(4, synth.CFG4, synth.CFG4_NKV)
    ref = _ref(case)
    dev = to_device(case)
    for blk in synth.CFG4_BLOCKS:
        S = -(-synth.CFG4.max_ctx // blk)
        say(f"hd256 blk={blk} S={S}")
        out, rec = run_gpu(case, S, blk, dev=dev)
        parity(out, ref, f"hd256 blk={blk}")
        check_records(rec, _records(case, S, blk), f"hd256 blk={blk}")


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
            parity(out, ref, f"growing nkv={nkv} S={S} blk={blk}")


def test_ragged_batch_sampled():
    """32 sequences, 32q/8kv hd 128, nkv_b ~ U{512..32768}: full-size launch,
    oracle on a sample of sequences (shortest, longest and four more)."""
    import decode_attention_gqa_amd as skv
    sh = synth.CFG5
    lengths = synth.cfg5_lengths()
    case = synth.make_case(5, sh, lengths)
    S, blk = skv.pick_splits(sh.batch, sh.n_head, sh.n_kv_head, sh.head_dim,
                             sh.max_ctx, 256)
    say(f"ragged B=32 S={S}")
    out, rec = run_gpu(case, S, blk)
    pick = sorted({int(np.argmin(lengths)), int(np.argmax(lengths)), 0, 7, 19, 31})
    sub = synth.Case(synth.Shape(len(pick), sh.n_head, sh.n_kv_head, sh.head_dim,
                                 sh.max_ctx),
                     case.q[pick], case.k[pick], case.v[pick],
                     case.positions[pick], case.scale)
    parity(out[pick], _ref(sub), "ragged sample")
    # split bounds of every sequence, bit-exact
    for b in range(sh.batch):
        lo, hi = oracle.split_bounds(int(lengths[b]), S, blk)
        lohi = rec[b, :, 0, 2:4].copy().view(np.int32)
        assert np.array_equal(lohi[:, 0], lo) and np.array_equal(lohi[:, 1], hi)


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
        parity(out, ref, f"precision hd={hd} S={S}")
        check_records(rec, _records(case, S), f"precision hd={hd} S={S}")


def test_deterministic():
    case = synth.make_case(2, synth.CFG2, 1500)
    dev = to_device(case)
    say("determinism")
    a, _ = run_gpu(case, 32, dev=dev)
    b, _ = run_gpu(case, 32, dev=dev)
    assert np.array_equal(a, b)
