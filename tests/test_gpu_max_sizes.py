"""GPU: the largest shapes the C ABI accepts, checked against closed forms.

The oracle's own pins fix these identities ("10 · R4 — decode split-attention
dim-parallel rewrite", section 2.1: the softmax-weighted mean over the live
rows, with the split merge exact): with every score equal, the output is the
plain mean of V over the live rows; with one row scoring 64 natural-log units
above all others, the output is that row's V to within e^-64 times the row
count; with one live row it is V[0] exactly. At these sizes the oracle would
need minutes on one core, so the expected values are those closed forms,
evaluated in fp64 from the definition of the synthetic data.

- One sequence whose K and V slices come within one tile of the 4 GiB limit of
  include/splitkv.h (head_dim 256, one KV head, 8,388,543 rows: row bases
  near 4 GiB), in one split (buffer record limits above 2 GiB), at the
  heuristic's split count and at the largest one (65,535, the last splits
  idle).
- 65,535 sequences (the largest batch) of one or no live row.
"""
import numpy as np
import pytest

from gpu_util import parity, say, torch_mod

pytestmark = pytest.mark.gpu

HD = 256
ROW_BYTES = HD * 2                      # one KV head
MAX_CTX = (1 << 32) // ROW_BYTES - 64 - 1   # (max_ctx + 64) rows below 4 GiB
PERIOD = 13


def _v_row_values(j):
    """V[j][d] = ((j mod 13) - 6) / 8 + (d mod 5) / 16, exact in fp16."""
    d = np.arange(HD)
    return ((j % PERIOD) - 6) / 8.0 + (d % 5) / 16.0


def _uniform_mean(nkv):
    """Mean over rows 0..nkv-1 of V (fp64): full periods of (j mod 13) - 6
    sum to zero, the remaining m rows to m(m-1)/2 - 6m."""
    m = nkv % PERIOD
    rows = (m * (m - 1) / 2.0 - 6.0 * m) / 8.0 / nkv
    return rows + (np.arange(HD) % 5) / 16.0


def _fill_v(torch, v):
    """Write the periodic V pattern into v [1][MAX_CTX][1][HD] on the device
    without a temporary of the cache's size."""
    tile = torch.tensor(np.stack([_v_row_values(j) for j in range(PERIOD)]),
                        dtype=torch.float16, device="cuda")
    flat = v.view(MAX_CTX, HD)
    full = MAX_CTX // PERIOD * PERIOD
    flat[:full].view(-1, PERIOD, HD).copy_(tile.expand(full // PERIOD, PERIOD, HD))
    flat[full:].copy_(tile[:MAX_CTX - full])


def test_largest_cache_slice():
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    nh, nkvh = 8, 1
    assert (MAX_CTX + 64) * nkvh * HD * 2 < (1 << 32)
    if torch.cuda.get_device_properties(0).total_memory < (12 << 30):
        pytest.skip("needs 12 GiB of device memory (two 4 GiB caches)")
    say(f"max sizes: K/V caches of {MAX_CTX} rows x {ROW_BYTES} B")
    k = torch.zeros((1, MAX_CTX, nkvh, HD), dtype=torch.float16, device="cuda")
    v = torch.empty_like(k)
    _fill_v(torch, v)
    # queries 1/16 everywhere and one needle row of ones: its score is
    # scale * 256 / 16 = 64 natural-log units for every head, all others 0
    needle = MAX_CTX - 3
    k[0, needle, 0, :] = 1.0
    q = torch.full((1, nh, HD), 1.0 / 16.0, device="cuda")
    scale = 4.0
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((1, nh, HD), device="cuda")
    S_h, blk = skv.pick_splits(1, nh, nkvh, HD, MAX_CTX,
                               torch.cuda.get_device_properties(0).multi_processor_count)
    for S in (1, S_h, 65535):
        part = torch.empty(skv.partials_bytes(1, nh, HD, S) // 4, device="cuda")
        for p, what in ((MAX_CTX - 1, "needle live"), (10**9, "clamped"),
                        (MAX_CTX - 10, "needle past the live rows")):
            say(f"max sizes: S={S} positions={p} ({what})")
            pos.fill_(p)
            out.fill_(float("nan"))
            skv.decode_attn(q, k, v, pos, part, out, S, 0, scale)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            nkv = min(p + 1, MAX_CTX)
            if needle < nkv:
                want = np.tile(_v_row_values(needle), (1, nh, 1))
            else:
                want = np.tile(_uniform_mean(nkv), (1, nh, 1))
            parity(got, want, f"max sizes S={S} {what}", "max sizes (closed forms)")
        del part
    del k, v
    torch.cuda.empty_cache()


def test_largest_batch():
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    B, nh, nkvh, hd, max_ctx = 65535, 2, 1, 64, 2
    rng = np.random.default_rng(7)
    v_host = rng.standard_normal((B, max_ctx, nkvh, hd)).astype(np.float16)
    k_host = rng.standard_normal((B, max_ctx, nkvh, hd)).astype(np.float16)
    q_host = rng.standard_normal((B, nh, hd)).astype(np.float32)
    # every third sequence is empty, the others have one live row
    pos_host = np.where(np.arange(B) % 3 == 0, -1, 0).astype(np.int32)
    dev = [torch.from_numpy(a).cuda() for a in (q_host, k_host, v_host, pos_host)]
    out = torch.full((B, nh, hd), float("nan"), device="cuda")
    for S in (1, 2):
        part = torch.empty(skv.partials_bytes(B, nh, hd, S) // 4, device="cuda")
        say(f"max batch: B={B} S={S}")
        skv.decode_attn(dev[0], dev[1], dev[2], dev[3], part, out, S, 0, 0.125)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        # one live row: p = 1 and the output is V[b][0] exactly; none: 0
        want = np.repeat(v_host[:, 0, :, :].astype(np.float32), nh, axis=1)
        want[pos_host < 0] = 0.0
        assert np.array_equal(got, want), f"max batch S={S}"
        del part
