"""GPU: the combine kernel alone on oracle records, and hipGraph replay of the
static grid as the live length grows ("10 · R4 — decode split-attention
dim-parallel rewrite", section 2.2: the grid is frozen at capture and the live
length is read from positions[] on the device, idle splits contribute zero).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import pack_records, parity, say, to_device, torch_mod

pytestmark = pytest.mark.gpu


def _combine_case(seed, B, S, nh, hd, idle_frac):
    rng = np.random.default_rng(seed)
    rec = np.zeros((B, S, nh, 4 + hd))
    rec[..., 0] = rng.uniform(-50, 50, (B, S, nh))
    rec[..., 1] = rng.uniform(0.5, 300, (B, S, nh))
    rec[..., 4:] = rng.standard_normal((B, S, nh, hd)) * rec[..., 1:2]
    idle = rng.random((B, S, nh)) < idle_frac
    rec[..., 0][idle] = -np.inf
    rec[..., 1][idle] = 0.0
    rec[..., 4:][idle] = 0.0
    rec[0, :, 0] = 0.0                    # one head with every split idle
    rec[0, :, 0, 0] = -np.inf
    return rec


@pytest.mark.parametrize("hd", [8, 16, 32, 64, 128, 256])
def test_combine_alone(hd):
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    for S, idle in ((1, 0.0), (5, 0.3), (64, 0.5), (263, 0.9)):
        B, nh = 2, 6
        rec = _combine_case(hd * 1000 + S, B, S, nh, hd, idle).astype(np.float32)
        want = oracle.combine(rec.astype(np.float64))
        part = torch.from_numpy(pack_records(rec)).cuda()
        out = torch.full((B, nh, hd), float("nan"), device="cuda")
        say(f"combine hd={hd} S={S}")
        skv.combine(part, out, S)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got[0, 0], np.zeros(hd, np.float32))
        parity(got, want, f"combine hd={hd} S={S}", "combine alone")


def test_graph_replay_growing_context():
    """Capture L layers of (partial + combine) once at nkv = 1, then replay
    with positions[] stepped; every replay matches the oracle and the eager
    call, and nkv = 1 reproduces V[0] exactly."""
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    sh = synth.CFG3
    layers = 3
    cases = [synth.make_offset_case(3, sh, sh.max_ctx, layer=l)
             for l in range(layers)]
    devs = [to_device(c) for c in cases]
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    S, blk = skv.pick_splits(1, sh.n_head, sh.n_kv_head, sh.head_dim, sh.max_ctx,
                             torch.cuda.get_device_properties(0).multi_processor_count)
    nbytes = skv.partials_bytes(1, sh.n_head, sh.head_dim, S)
    parts = [torch.empty(nbytes // 4, device="cuda") for _ in range(layers)]
    outs = [torch.empty((1, sh.n_head, sh.head_dim), device="cuda")
            for _ in range(layers)]

    def step():
        for l in range(layers):
            q, k, v, _ = devs[l]
            skv.decode_attn(q, k, v, pos, parts[l], outs[l], S, blk, cases[l].scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"graph capture S={S} blk={blk}")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for nkv in (1, 2, 127, 128, 129, 1000, 4097, 16385, 32769, 5, 1):
        pos.fill_(nkv - 1)
        say(f"graph replay nkv={nkv}")
        graph.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy().copy() for o in outs]
        step()                                   # eager call, same inputs
        torch.cuda.synchronize()
        for l in range(layers):
            assert np.array_equal(got[l], outs[l].cpu().numpy()), (nkv, l)
            c = cases[l]
            c.positions[:] = nkv - 1
            ref = oracle.decode_attn(c.q, c.k, c.v, c.positions, sh.n_kv_head,
                                     c.scale)
            parity(got[l], ref, f"replay nkv={nkv} layer={l}",
                   "3 growing, graph replays")
            if nkv == 1:
                for h in range(sh.n_head):
                    assert np.array_equal(
                        got[l][0, h], c.v[0, 0, h // sh.group].astype(np.float32))
