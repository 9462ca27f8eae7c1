"""Helpers for the GPU parity tests: move a synthetic case to the device, run
the HIP path through the C ABI, and compare with the oracle element by element.

Parity bar (per element): |gpu - oracle| <= 5e-5, or <= 1e-3 * |oracle|. Integer
outputs (split bounds) must be bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np

ABS_TOL = 5e-5
REL_TOL = 1e-3

# Worst errors seen per workload over the session: {label: [max abs, max rel,
# elements compared]}. conftest.py prints the table at the end of the run and,
# when SPLITKV_PARITY_LOG names a file, writes it there as JSON.
WORST: dict = {}


def records_view(buf, B, S, NH, hd):
    """The library's records buffer (flat float32: the output sums of every
    record [B][S][NH][hd], then the headers {mx, S, lo, hi} [B][NH][S][4]) as
    one array [B][S][NH][4 + hd] of records {mx, S, lo, hi, oc[0..hd)}, the
    layout the oracle uses."""
    buf = np.asarray(buf).reshape(-1)
    n_oc = B * S * NH * hd
    oc = buf[:n_oc].reshape(B, S, NH, hd)
    hdr = buf[n_oc:n_oc + B * NH * S * 4].reshape(B, NH, S, 4)
    return np.concatenate([hdr.transpose(0, 2, 1, 3), oc], axis=-1)


def pack_records(rec):
    """Inverse of records_view: records [B][S][NH][4 + hd] to the flat buffer."""
    rec = np.asarray(rec)
    return np.concatenate([rec[..., 4:].reshape(-1),
                           rec[..., :4].transpose(0, 2, 1, 3).reshape(-1)])


def say(*parts):
    """Name the case about to run on the GPU, flushed, so a crash log shows it."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch


def to_device(case):
    torch = torch_mod()
    dev = torch.device("cuda", 0)
    q = torch.from_numpy(np.ascontiguousarray(case.q)).to(dev)
    k = torch.from_numpy(np.ascontiguousarray(case.k)).to(dev)
    v = torch.from_numpy(np.ascontiguousarray(case.v)).to(dev)
    pos = torch.from_numpy(np.ascontiguousarray(case.positions, np.int32)).to(dev)
    return q, k, v, pos


def alloc_outputs(shape, n_splits):
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    nbytes = skv.partials_bytes(shape.batch, shape.n_head, shape.head_dim,
                                n_splits)
    part = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    part.fill_(float("nan"))   # every record must be written by the kernel
    out = torch.empty((shape.batch, shape.n_head, shape.head_dim),
                      dtype=torch.float32, device="cuda")
    out.fill_(float("nan"))
    return part, out


def run_gpu(case, n_splits, block_len=0, dev=None):
    """decode_attn through the C ABI; returns (out, records) as numpy."""
    import decode_attention_gqa_amd as skv
    torch = torch_mod()
    sh = case.shape
    q, k, v, pos = dev if dev is not None else to_device(case)
    part, out = alloc_outputs(sh, n_splits)
    skv.decode_attn(q, k, v, pos, part, out, n_splits, block_len, case.scale)
    torch.cuda.synchronize()
    rec = records_view(part.cpu().numpy(), sh.batch, n_splits, sh.n_head,
                       sh.head_dim)
    return out.cpu().numpy(), rec


def parity(got, ref, what="", cfg=None):
    """Assert the parity bar; returns (max abs err, max rel err). With `cfg`
    (a workload label) the errors also count towards that workload's worst
    case in WORST. The relative error is taken over elements with
    |oracle| > 1e-6."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN in GPU output"
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    ok = (err <= ABS_TOL) | (err <= REL_TOL * np.abs(ref))
    if not ok.all():
        idx = np.unravel_index(np.argmax(np.where(ok, 0, err)), err.shape)
        raise AssertionError(
            f"{what}: {int((~ok).sum())} of {ok.size} outside the bar; worst at "
            f"{idx}: gpu {got[idx]!r} oracle {ref[idx]!r} abs {err[idx]:.3e}")
    worst_abs = float(err.max()) if err.size else 0.0
    worst_rel = float(np.where(np.abs(ref) > 1e-6, rel, 0).max()) \
        if rel.size else 0.0
    if cfg is not None:
        w = WORST.setdefault(cfg, [0.0, 0.0, 0])
        w[0] = max(w[0], worst_abs)
        w[1] = max(w[1], worst_rel)
        w[2] += int(err.size)
    return worst_abs, worst_rel


def check_records(rec_gpu, rec_ref, what="", cfg=None):
    """Records: lo/hi bit-exact, idle slots exact, mx / S / oc/S within the bar."""
    lohi = rec_gpu[..., 2:4].copy().view(np.int32)
    assert np.array_equal(lohi, rec_ref[..., 2:4].astype(np.int32)), \
        f"{what}: split bounds differ"
    idle = rec_ref[..., 0] == -np.inf
    assert np.array_equal(rec_gpu[..., 0] == -np.inf, idle), \
        f"{what}: idle pattern differs"
    assert np.all(rec_gpu[..., 1][idle] == 0.0)
    assert np.all(rec_gpu[..., 4:][idle] == 0.0)
    live = ~idle
    if live.any():
        rc = None if cfg is None else cfg + " records"
        parity(rec_gpu[..., 0][live], rec_ref[..., 0][live], what + " mx", rc)
        parity(rec_gpu[..., 1][live], rec_ref[..., 1][live], what + " S", rc)
        parity(rec_gpu[..., 4:][live] / rec_gpu[..., 1][live][:, None],
               rec_ref[..., 4:][live] / rec_ref[..., 1][live][:, None],
               what + " oc/S", rc)
