"""GPU: the per-query-head grid (one workgroup per split and query head, the
launch shape of "10 · R4", section 3.2, and of the Red Lite kernel before
grouping) against the grouped kernel and the oracle.

Each query head's arithmetic is the same in both forms (its own MFMA column,
its own running max and sum), so the records must be equal bit for bit; the
combined output must meet the parity bar against the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (alloc_outputs, parity, records_view, say, to_device,
                      torch_mod)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_per_head_equals_grouped(hd):
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    for G in (1, 2, 4, 7, 8):
        nkvh = 2
        sh = synth.Shape(2, G * nkvh, nkvh, hd, 700)
        case = synth.make_case(40 + G, sh, np.array([700, 333]),
                               poison_tail=True)
        dev = to_device(case)
        q, k, v, pos = dev
        want = oracle.decode_attn(case.q, case.k, case.v, case.positions,
                                  nkvh, case.scale)
        for S, blk in ((1, 0), (5, 0), (33, 0), (6, 128)):
            pa, out = alloc_outputs(sh, S)
            pb, _ = alloc_outputs(sh, S)
            say(f"per-head hd={hd} G={G} S={S} blk={blk}")
            skv.partial(q, k, v, pos, pa, S, blk, case.scale)
            skv.partial_per_head(q, k, v, pos, pb, S, blk, case.scale)
            skv.combine(pb, out, S)
            torch.cuda.synchronize()
            ra = records_view(pa.cpu().numpy(), sh.batch, S, sh.n_head, hd)
            rb = records_view(pb.cpu().numpy(), sh.batch, S, sh.n_head, hd)
            diff = ra.view(np.uint32) != rb.view(np.uint32)
            if diff.any():
                idx = np.argwhere(diff)
                heads = sorted({int(i[2]) for i in idx})
                fields = sorted({int(min(i[3], 4)) for i in idx})
                fin = np.isfinite(ra) & np.isfinite(rb)
                mad = float(np.max(np.abs(ra - rb)[fin & diff])) if \
                    (fin & diff).any() else float("nan")
                raise AssertionError(
                    f"hd={hd} G={G} S={S} blk={blk}: {int(diff.sum())} words "
                    f"differ; heads {heads}; fields {fields} (4 = oc); max "
                    f"abs diff {mad:.3e}; first {idx[0].tolist()} grouped "
                    f"{ra[tuple(idx[0])]!r} per-head {rb[tuple(idx[0])]!r}")
            parity(out.cpu().numpy(), want, f"per-head hd={hd} G={G} S={S}",
                   "per-query-head grid")
