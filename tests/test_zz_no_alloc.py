"""GPU: the allocation-free entry point (splitkv_decode_attn_noalloc, for
callers that cannot allocate device memory) against splitkv_decode_attn with a
caller records buffer, through the C ABI. Two calls in a row share the
library's device scratch, the second with a smaller input; each output must be
bit-identical to the existing entry point's (the same kernels), and within the
parity bar of it.
"""
import numpy as np
import pytest

import synth
from gpu_util import alloc_outputs, parity, say, to_device, torch_mod

pytestmark = pytest.mark.gpu


def _both(case, S, blk=0):
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    q, k, v, pos = to_device(case)
    part, out_ref = alloc_outputs(case.shape, S)
    skv.decode_attn(q, k, v, pos, part, out_ref, S, blk, case.scale)
    out = torch.full_like(out_ref, float("nan"))
    skv.decode_attn_noalloc(q, k, v, pos, out, S, blk, case.scale)
    torch.cuda.synchronize()
    return out.cpu().numpy(), out_ref.cpu().numpy()


def test_noalloc_matches_decode_attn_two_calls():
    import decode_attention_gqa_amd as skv
    # first call: the headline shape at 32K rows, 128 splits (1.9 MB of
    # records); second call: the tiny workload (4 splits, 4 KB), so that it
    # runs over the larger call's leftover records
    big = synth.make_case(3, synth.Shape(1, 28, 4, 128, 33024), 32768,
                          poison_tail=True)
    S_big, blk_big = skv.pick_splits(1, 28, 4, 128, 33024, 256)
    say(f"noalloc call 1: 28q/4kv hd128 nkv 32768 S={S_big}")
    got, want = _both(big, S_big, blk_big)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    parity(got, want, "noalloc call 1")
    small = synth.make_case(1, synth.CFG1, 256, poison_tail=True)
    say(f"noalloc call 2: 4q/2kv hd64 nkv 256 S={synth.CFG1_SPLITS}")
    got, want = _both(small, synth.CFG1_SPLITS)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    parity(got, want, "noalloc call 2")


def test_noalloc_rejects_oversize_records():
    """Records beyond the scratch: an error status, nothing enqueued."""
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    case = synth.make_case(1, synth.CFG1, 256)
    q, k, v, pos = to_device(case)
    out = torch.zeros((1, 4, 64), device="cuda")
    per_split = skv.partials_bytes(1, 4, 64, 1)
    S = skv.NOALLOC_SCRATCH_BYTES // per_split + 1
    say(f"noalloc oversize S={S}")
    with pytest.raises(skv.SplitKVError) as e:
        skv.decode_attn_noalloc(q, k, v, pos, out, S, 0, case.scale)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_noalloc_in_a_graph_matches_decode_attn():
    """The use this entry point is for: captured in a hipGraph (after one
    call outside capture on the device), then replayed as the context grows.
    Every replay's output is bit-identical to splitkv_decode_attn on the same
    inputs, with eager calls of both entry points between the replays."""
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    sh = synth.Shape(1, 28, 4, 128, 4096)
    case = synth.make_case(3, sh, 4096)
    q, k, v, _ = to_device(case)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    S, blk = skv.pick_splits(1, 28, 4, 128, 4096, 256)
    out = torch.full((1, 28, 128), float("nan"), device="cuda")
    part, out_ref = alloc_outputs(sh, S)

    def step():
        skv.decode_attn_noalloc(q, k, v, pos, out, S, blk, case.scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # first call outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"noalloc graph capture S={S}")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for nkv in (1, 17, 1000, 4096, 300):
        pos.fill_(nkv - 1)
        say(f"noalloc graph replay nkv={nkv}")
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy().copy()
        skv.decode_attn(q, k, v, pos, part, out_ref, S, blk, case.scale)
        step()                                   # eager noalloc between replays
        torch.cuda.synchronize()
        want = out_ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), nkv
        assert np.array_equal(out.cpu().numpy().view(np.uint32),
                              want.view(np.uint32)), nkv
