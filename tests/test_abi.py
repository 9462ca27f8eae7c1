"""C-ABI checks that need no GPU: the library loads, exports every symbol the
headers declare, reports sizes, runs the split heuristic, and rejects every
bad argument with its status code before any HIP call.
"""
import ctypes
import glob
import os
import re

import pytest

import decode_attention_gqa_amd as skv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, EUNSUP, EALIGN, ELAUNCH, ESCRATCH = 0, -1, -2, -3, -4, -5


def _declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(splitkv_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib(splitkv_lib_path):
    return skv.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared_symbols()
    assert "splitkv_decode_attn" in declared and len(declared) >= 9
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(skv.SIGNATURES)


def test_version_and_strerror(lib):
    assert lib.splitkv_abi_version() == 3
    texts = {c: skv.strerror(c)
             for c in (OK, EINVAL, EUNSUP, EALIGN, ELAUNCH, ESCRATCH)}
    assert len(set(texts.values())) == 6
    assert skv.strerror(-99) == "unknown status"


def test_partials_bytes(lib):
    # batch * n_splits * n_head * (4 + hd) * 4
    assert skv.partials_bytes(1, 28, 128, 32) == 32 * 28 * 132 * 4
    assert skv.partials_bytes(32, 32, 128, 7) == 32 * 7 * 32 * 132 * 4
    assert skv.partials_bytes(0, 28, 128, 32) == 0
    assert skv.partials_bytes(1, 28, 128, -1) == 0


def test_pick_splits_properties(lib):
    for shape in [(1, 28, 4, 128, 2048), (1, 28, 4, 128, 33024),
                  (1, 16, 2, 256, 8400), (32, 32, 8, 128, 32768),
                  (1, 4, 2, 64, 256), (1, 4, 2, 8, 1024)]:
        B, nh, nkvh, hd, T = shape
        S, blk = skv.pick_splits(*shape, cu_count=256)
        assert 1 <= S <= 65535 and blk >= 0
        if blk:
            assert blk * S >= T
        # never so many splits that a full-length split is under one tile
        assert S == 1 or T // S >= 32
    # Values the rule gives on 256 compute units. One sequence: one full round
    # of resident workgroups (2 per compute unit at hd128 -> 128 splits over 4
    # KV heads; 1 at hd256 -> 128 over 2), capped so a full-length split
    # keeps one 32-row tile (2048 / 32 -> 64; 256 / 32 -> 8), and at hd256
    # (8 waves) at the splits whose full length fills one 16-row tile per
    # wave (ceil(8400 / 128) -> 66). Batches: ~16 workgroups per compute
    # unit, splits of >= 1024 rows.
    cases = {(1, 28, 4, 128, 33024): 128, (1, 28, 4, 128, 2048): 64,
             (1, 16, 2, 256, 8400): 66, (1, 16, 2, 256, 33024): 128,
             (32, 32, 8, 128, 32768): 16,
             (16, 32, 8, 128, 32768): 32, (8, 32, 8, 128, 32768): 32,
             (4, 32, 8, 128, 32768): 32, (32, 32, 8, 128, 4096): 4,
             (1, 4, 2, 64, 256): 8, (1, 28, 4, 128, 40): 1,
             (1, 24, 3, 128, 33024): 170}
    for shape, want in cases.items():
        assert skv.pick_splits(*shape, cu_count=256) == (want, 0), shape
    # never more than one round of resident workgroups for one sequence
    for hd in (8, 16, 32, 64, 128, 256):
        for g in range(1, 9):
            for nkvh in (1, 2, 3, 4, 5, 8):
                S, _ = skv.pick_splits(1, g * nkvh, nkvh, hd, 1 << 16, 256)
                assert S * nkvh <= skv.workgroups_per_cu(hd, g) * 256, (hd, g)
    with pytest.raises(skv.SplitKVError):
        skv.pick_splits(1, 28, 5, 128, 2048, 256)      # 28 % 5 != 0
    with pytest.raises(skv.SplitKVError):
        skv.pick_splits(1, 28, 4, 96, 2048, 256)       # head_dim not compiled
    with pytest.raises(skv.SplitKVError):
        skv.pick_splits(1, 28, 4, 128, 2048, 0)        # no compute units


def test_pick_splits_rows(lib):
    # one row: the one-row rule
    for shape in [(1, 28, 4, 128, 2048), (1, 28, 4, 128, 33024),
                  (1, 16, 2, 256, 8400), (32, 32, 8, 128, 32768),
                  (1, 4, 2, 64, 256), (1, 4, 2, 8, 1024)]:
        B, nh, nkvh, hd, T = shape
        assert (skv.pick_splits_rows(B, 1, nh, nkvh, hd, T, 256) ==
                skv.pick_splits(*shape, cu_count=256)), shape
    # Workgroups per split = KV heads x sequences x blocks of rows; rows share
    # a block when their (row, head) pairs fit the MFMA columns (16 at hd 64
    # and 128, 8 at hd 256): G = 7 at hd128 takes 2 rows per block, G = 4
    # four, G = 2 eight, G = 8 at hd256 one, G = 1 eight, and the vector-ALU
    # head sizes one. One round of 2 (hd128) / 1 (hd256) resident
    # workgroups per compute unit on 256 units; hd32 G = 2: 3 per unit,
    # capped at max_ctx / 32 splits.
    cases = {(1, 2, 28, 4, 128, 33024): 128,    # 1 block  x 4 heads
             (1, 4, 28, 4, 128, 33024): 64,     # 2 blocks x 4
             (1, 8, 28, 4, 128, 33024): 32,     # 4 blocks x 4
             (1, 3, 28, 4, 128, 33024): 64,     # 2 blocks (last half full)
             (1, 2, 16, 2, 256, 8400): 64,      # 2 blocks x 2, 1 per unit
             (1, 8, 8, 8, 128, 32768): 64,      # 1 block  x 8
             (2, 2, 28, 4, 128, 32768): 64,     # 2 sequences, 8 units
             (1, 4, 32, 8, 128, 32768): 64,     # G 4: 4 rows in 1 block x 8
             (1, 8, 32, 8, 128, 32768): 32,     # 2 blocks x 8
             (1, 8, 16, 8, 128, 32768): 64,     # G 2: 8 rows in 1 block x 8
             (1, 4, 32, 8, 256, 32768): 16,     # hd256 G 4: 2 per block, 1/unit
             (1, 4, 4, 2, 32, 1024): 32}        # 4 rows x 2, capped
    for (B, n_q, nh, nkvh, hd, T), want in cases.items():
        assert skv.pick_splits_rows(B, n_q, nh, nkvh, hd, T, 256) == \
            (want, 0), (B, n_q, nh, nkvh, hd, T)
    with pytest.raises(skv.SplitKVError):
        skv.pick_splits_rows(1, 0, 28, 4, 128, 2048, 256)   # no rows


# Fake, aligned addresses: every case below must fail validation, so nothing
# is ever dereferenced or launched. As a second guard these cases only run on
# hosts without a GPU, where a launch could not reach a device anyway.
A = 0x10000


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


cpu_only = pytest.mark.skipif(_has_gpu(), reason="raw-pointer validation "
                              "cases run on GPU-less hosts only")


def _partial_args(**over):
    args = dict(q=A, k=A + 0x1000, v=A + 0x2000, pos=A + 0x3000,
                part=A + 0x4000, B=1, nh=28, nkvh=4, hd=128, T=2048, S=32,
                blk=0, scale=0.088)
    args.update(over)
    return args


def _call_partial(lib, a):
    return lib.splitkv_partial(a["q"], a["k"], a["v"], a["pos"], a["part"],
                               a["B"], a["nh"], a["nkvh"], a["hd"], a["T"],
                               a["S"], a["blk"], a["scale"], None)


def _call_decode(lib, a, out=A + 0x5000):
    return lib.splitkv_decode_attn(a["q"], a["k"], a["v"], a["pos"], a["part"],
                                   out, a["B"], a["nh"], a["nkvh"], a["hd"],
                                   a["T"], a["S"], a["blk"], a["scale"], None)


BAD_PARTIAL = [
    ("null q", dict(q=0), EINVAL),
    ("null k", dict(k=0), EINVAL),
    ("null v", dict(v=0), EINVAL),
    ("null positions", dict(pos=0), EINVAL),
    ("null partials", dict(part=0), EINVAL),
    ("batch 0", dict(B=0), EINVAL),
    ("n_head 0", dict(nh=0), EINVAL),
    ("n_kv_head 0", dict(nkvh=0), EINVAL),
    ("max_ctx 0", dict(T=0), EINVAL),
    ("n_splits 0", dict(S=0), EINVAL),
    ("n_splits too big", dict(S=65536), EINVAL),
    ("negative block_len", dict(blk=-1), EINVAL),
    ("heads not divisible", dict(nkvh=3), EINVAL),
    ("block rule too short", dict(S=8, blk=128), EINVAL),
    ("block rule overflow", dict(S=65535, blk=1 << 20), EINVAL),
    ("max_ctx near int max", dict(T=2**31 - 10, nh=1, nkvh=1, hd=8, S=16),
     EINVAL),
    ("sequence cache >= 4 GiB", dict(T=2**24, nh=1, nkvh=1, hd=128), EINVAL),
    ("non-finite scale", dict(scale=float("inf")), EINVAL),
    ("nan scale", dict(scale=float("nan")), EINVAL),
    ("head_dim 96", dict(hd=96), EUNSUP),
    ("head_dim 512", dict(hd=512), EUNSUP),
    ("group 9", dict(nh=36, nkvh=4), EUNSUP),
    ("q misaligned", dict(q=A + 4), EALIGN),
    ("k misaligned", dict(k=A + 0x1000 + 2), EALIGN),
    ("v misaligned", dict(v=A + 0x2000 + 8), EALIGN),
    ("partials misaligned", dict(part=A + 0x4000 + 4), EALIGN),
    ("positions misaligned", dict(pos=A + 0x3000 + 2), EALIGN),
]


@cpu_only
@pytest.mark.parametrize("what,over,code", BAD_PARTIAL,
                         ids=[c[0] for c in BAD_PARTIAL])
def test_partial_rejects(lib, what, over, code):
    a = _partial_args(**over)
    assert _call_partial(lib, a) == code
    assert _call_decode(lib, a) == code


@cpu_only
@pytest.mark.parametrize("what,over,code", BAD_PARTIAL + [
    ("head_dim 32 (vector-ALU family)", dict(hd=32), EUNSUP)],
    ids=[c[0] for c in BAD_PARTIAL] + ["head_dim 32"])
def test_partial_per_head_rejects(lib, what, over, code):
    a = _partial_args(**over)
    assert lib.splitkv_partial_per_head(
        a["q"], a["k"], a["v"], a["pos"], a["part"], a["B"], a["nh"],
        a["nkvh"], a["hd"], a["T"], a["S"], a["blk"], a["scale"], None) == code


@cpu_only
def test_decode_rejects_bad_out(lib):
    a = _partial_args()
    assert _call_decode(lib, a, out=0) == EINVAL
    assert _call_decode(lib, a, out=A + 0x5000 + 4) == EALIGN


def _call_noalloc(lib, a, out=A + 0x5000):
    return lib.splitkv_decode_attn_noalloc(
        a["q"], a["k"], a["v"], a["pos"], out, a["B"], a["nh"], a["nkvh"],
        a["hd"], a["T"], a["S"], a["blk"], a["scale"], None)


@cpu_only
@pytest.mark.parametrize(
    "what,over,code",
    [c for c in BAD_PARTIAL if c[0] not in ("null partials",
                                            "partials misaligned")],
    ids=[c[0] for c in BAD_PARTIAL if c[0] not in ("null partials",
                                                   "partials misaligned")])
def test_decode_noalloc_rejects(lib, what, over, code):
    """The allocation-free entry point validates like decode_attn (it has no
    partials argument), before any HIP call."""
    assert _call_noalloc(lib, _partial_args(**over)) == code


@cpu_only
def test_decode_noalloc_rejects_bad_out_and_oversize(lib):
    a = _partial_args()
    assert _call_noalloc(lib, a, out=0) == EINVAL
    assert _call_noalloc(lib, a, out=A + 0x5000 + 4) == EALIGN
    cap = skv.NOALLOC_SCRATCH_BYTES
    # records of 28 heads x (4 + 128) floats per split: 1,134 splits fit
    per_split = skv.partials_bytes(1, 28, 128, 1)
    s_max = cap // per_split
    assert s_max == 1134
    assert _call_noalloc(lib, _partial_args(S=s_max + 1, T=65536)) == ESCRATCH
    # 32 sequences of 32q hd128: 31 splits fit, 32 do not
    big = dict(B=32, nh=32, nkvh=8, T=32768)
    assert skv.partials_bytes(32, 32, 128, 31) <= cap < \
        skv.partials_bytes(32, 32, 128, 32)
    assert _call_noalloc(lib, _partial_args(S=32, **big)) == ESCRATCH


def _call_step(lib, a, kn=A + 0x6000, vn=A + 0x7000, out=A + 0x5000):
    return lib.splitkv_decode_step(a["q"], kn, vn, a["k"], a["v"], a["pos"],
                                   a["part"], out, a["B"], a["nh"], a["nkvh"],
                                   a["hd"], a["T"], a["S"], a["blk"],
                                   a["scale"], None)


@cpu_only
@pytest.mark.parametrize("what,over,code", BAD_PARTIAL,
                         ids=[c[0] for c in BAD_PARTIAL])
def test_decode_step_rejects(lib, what, over, code):
    """The folded decode step validates like decode_attn, before any
    launch."""
    assert _call_step(lib, _partial_args(**over)) == code


@cpu_only
def test_decode_step_rejects_bad_new_rows(lib):
    a = _partial_args()
    assert _call_step(lib, a, kn=0) == EINVAL
    assert _call_step(lib, a, vn=0) == EINVAL
    assert _call_step(lib, a, kn=A + 0x6000 + 4) == EALIGN
    assert _call_step(lib, a, vn=A + 0x7000 + 8) == EALIGN
    assert _call_step(lib, a, out=0) == EINVAL


BAD_COMBINE = [
    ("null partials", (0, A + 0x100, 1, 28, 128, 32), EINVAL),
    ("null out", (A, 0, 1, 28, 128, 32), EINVAL),
    ("batch 0", (A, A + 0x100, 0, 28, 128, 32), EINVAL),
    ("n_head 0", (A, A + 0x100, 1, 0, 128, 32), EINVAL),
    ("n_splits 0", (A, A + 0x100, 1, 28, 128, 0), EINVAL),
    ("head_dim 48", (A, A + 0x100, 1, 28, 48, 32), EUNSUP),
    ("partials misaligned", (A + 4, A + 0x100, 1, 28, 128, 32), EALIGN),
    ("out misaligned", (A, A + 0x104, 1, 28, 128, 32), EALIGN),
    ("sequence records >= 2 GiB", (A, A + 0x100, 1, 8192, 256, 1024), EINVAL),
]


@cpu_only
@pytest.mark.parametrize("what,args,code", BAD_COMBINE,
                         ids=[c[0] for c in BAD_COMBINE])
def test_combine_rejects(lib, what, args, code):
    assert lib.splitkv_combine(*args, None) == code


@cpu_only
def test_probe_rejects(lib):
    assert lib.splitkv_probe_read(0, 16, A, 1, None) == EINVAL
    assert lib.splitkv_probe_read(A, 17, A + 0x100, 1, None) == EINVAL
    assert lib.splitkv_probe_read(A, 16, A + 0x100, 0, None) == EINVAL
    assert lib.splitkv_probe_read(A + 8, 16, A + 0x100, 1, None) == EALIGN
    assert lib.splitkv_probe_copy(A, A + 8, 32, 1, None) in (EINVAL, EALIGN)
    assert lib.splitkv_probe_copy(A, A + 16, 32, 1, None) == EINVAL  # overlap
    assert lib.splitkv_probe_copy(A, 0, 32, 1, None) == EINVAL


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        skv.load(str(tmp_path / "nope.so"))


BAD_APPEND = [
    ("null k_new", dict(kn=0), EINVAL),
    ("null v_new", dict(vn=0), EINVAL),
    ("null k_cache", dict(kc=0), EINVAL),
    ("null v_cache", dict(vc=0), EINVAL),
    ("null positions", dict(pos=0), EINVAL),
    ("batch 0", dict(B=0), EINVAL),
    ("n_rows 0", dict(n=0), EINVAL),
    ("n_rows too big", dict(n=65536), EINVAL),
    ("n_kv_head 0", dict(nkvh=0), EINVAL),
    ("max_ctx 0", dict(T=0), EINVAL),
    ("head_dim 96", dict(hd=96), EUNSUP),
    ("k_new misaligned", dict(kn=A + 4), EALIGN),
    ("v_cache misaligned", dict(vc=A + 0x3000 + 8), EALIGN),
    ("positions misaligned", dict(pos=A + 0x4000 + 2), EALIGN),
]


@cpu_only
@pytest.mark.parametrize("what,over,code", BAD_APPEND,
                         ids=[c[0] for c in BAD_APPEND])
def test_append_rejects(lib, what, over, code):
    a = dict(kn=A, vn=A + 0x1000, kc=A + 0x2000, vc=A + 0x3000, pos=A + 0x4000,
             B=2, n=1, nkvh=4, hd=128, T=2048)
    a.update(over)
    assert lib.splitkv_append_kv(a["kn"], a["vn"], a["kc"], a["vc"], a["pos"],
                                 a["B"], a["n"], a["nkvh"], a["hd"], a["T"],
                                 None) == code


@cpu_only
@pytest.mark.parametrize("what,over,code", BAD_PARTIAL + [
    ("n_q 0", dict(nq=0), EINVAL),
    ("batch * n_q too big", dict(B=300, nq=300), EINVAL),
    ("n_q * n_head too big", dict(nq=3000, nh=28), EINVAL)],
    ids=[c[0] for c in BAD_PARTIAL] + ["n_q 0", "grid z", "records per row"])
def test_rows_reject(lib, what, over, code):
    a = _partial_args(**{k: v for k, v in over.items() if k != "nq"})
    nq = over.get("nq", 2)
    assert lib.splitkv_partial_rows(
        a["q"], a["k"], a["v"], a["pos"], a["part"], a["B"], nq, a["nh"],
        a["nkvh"], a["hd"], a["T"], a["S"], a["blk"], a["scale"], None) == code
    assert lib.splitkv_decode_attn_rows(
        a["q"], a["k"], a["v"], a["pos"], a["part"], A + 0x5000, a["B"], nq,
        a["nh"], a["nkvh"], a["hd"], a["T"], a["S"], a["blk"], a["scale"],
        None) == code


def test_one_hip_runtime_whatever_the_import_order():
    """Loading the library before torch has been imported must not bring a
    second HIP runtime into the process (torch ships its own under the same
    soname): with two, kernels and streams belong to different runtimes and
    every launch fails."""
    import subprocess
    import sys
    code = (
        "import decode_attention_gqa_amd as skv\n"
        "skv.load()\n"
        "import torch\n"
        "maps = {l.split()[-1] for l in open('/proc/self/maps')\n"
        "        if 'libamdhip64' in l}\n"
        "print(len(maps))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, "-c", code], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert p.returncode == 0, p.stderr
    assert p.stdout.strip().splitlines()[-1] == "1", p.stdout
