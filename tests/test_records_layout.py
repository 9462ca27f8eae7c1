"""CPU: the tests' view of the library's split-records buffer follows the
layout that include/splitkv.h states (every record's output sums first,
[B][S][NH][hd], then every record's header {mx, S, lo, hi}, [B][NH][S][4])."""
import numpy as np

from gpu_util import pack_records, records_view


def test_records_view_places_fields_as_documented():
    B, S, NH, hd = 2, 3, 5, 8
    buf = np.arange(B * S * NH * (4 + hd), dtype=np.float32)
    rec = records_view(buf, B, S, NH, hd)
    assert rec.shape == (B, S, NH, 4 + hd)
    n_oc = B * S * NH * hd
    for b in range(B):
        for sp in range(S):
            for h in range(NH):
                for d in range(hd):
                    assert rec[b, sp, h, 4 + d] == buf[((b * S + sp) * NH + h) * hd + d]
                for f in range(4):
                    assert rec[b, sp, h, f] == buf[n_oc + ((b * NH + h) * S + sp) * 4 + f]
    assert np.array_equal(pack_records(rec), buf)
