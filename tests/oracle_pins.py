"""Pins of the fp64 oracle against what the pages and mathematics fix.

Every pin takes a loaded oracle library and raises AssertionError when the
oracle disagrees. None of them recomputes the oracle's own formula the same
way: the references are printed page values, closed forms, exact identities,
invariants, numpy library routines, and brute force in 40-digit decimal
arithmetic. ``test_oracle_pins.py`` runs them against the real oracle and
``test_oracle_mutants.py`` checks that each planted mistake in a copy of the
oracle fails at least one of them.

Pages: "10 · R4 — decode split-attention dim-parallel rewrite" (R4),
dotLLM issue #199 (#199), "Red Lite dev35 — long-context decode: grouped
split-K attention" (Red Lite).
"""
from __future__ import annotations

import decimal
import json
import math
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "page_examples.json")


def _case(seed, B, nh, nkvh, hd, max_ctx, nkv, q_scale=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, nh, hd)) * q_scale).astype(np.float32)
    k = rng.standard_normal((B, max_ctx, nkvh, hd)).astype(np.float16)
    v = rng.standard_normal((B, max_ctx, nkvh, hd)).astype(np.float16)
    pos = (np.broadcast_to(np.asarray(nkv), (B,)) - 1).astype(np.int32)
    return q, k, v, pos


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
def pin_f16_decoder(lib):
    """The oracle's binary16 decoder equals numpy's for all 65536 patterns."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = np.array([lib.oracle_f16_to_f64(int(b)) for b in bits])
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan), "NaN patterns differ"
    assert np.array_equal(ours[~nan], ref[~nan]), "finite/inf values differ"
    # signed zeros keep their sign
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def pin_live_length(lib):
    """R4 2.2: nkv = positions + 1; clamped to [0, max_ctx] (reading)."""
    L = lambda p, m: oracle.live_length(p, m, lib)  # noqa: E731
    assert L(0, 10) == 1 and L(9, 10) == 10 and L(5, 10) == 6
    assert L(-1, 10) == 0 and L(-7, 10) == 0
    assert L(10, 10) == 10 and L(2**31 - 1, 10) == 10
    assert L(-2**31, 10) == 0


def pin_split_bounds_pages(lib):
    """Rows per split printed on the pages (golden/page_examples.json)."""
    with open(GOLDEN) as f:
        gold = json.load(f)
    for ex in gold["split_rows"]:
        lo, hi = oracle.split_bounds(ex["nkv"], ex["n_splits"], ex["block_len"],
                                     lib)
        sizes = (hi - lo)[hi > lo]
        assert sizes[0] == ex["rows_per_split"], (ex["cite"], lo, hi)
        assert lo[0] == 0 and lo[1] == ex["rows_per_split"], ex["cite"]


def pin_split_bounds_partition(lib):
    """Brute force: live splits tile [0, nkv) in order with equal chunks."""
    for nkv in list(range(0, 70)) + [127, 128, 129, 255, 256, 257, 300]:
        for S in (1, 2, 3, 4, 5, 7, 8, 31, 32, 33, 40):
            for blk in (0, 1, 3, 16, 64, 128):
                if blk and blk * S < nkv:
                    continue
                lo, hi = oracle.split_bounds(nkv, S, blk, lib)
                chunk = blk if blk else -(-nkv // S)
                covered = []
                for sp in range(S):
                    assert lo[sp] == sp * chunk, (nkv, S, blk, sp)
                    assert hi[sp] == min(nkv, sp * chunk + chunk), (nkv, S, blk)
                    covered.extend(range(lo[sp], hi[sp]))
                assert covered == list(range(nkv)), (nkv, S, blk)


def pin_bruteforce_decimal(lib):
    """Tiny inputs: softmax without max subtraction in 40-digit decimals."""
    ctx = decimal.Context(prec=40)
    D = lambda x: decimal.Decimal(float(x))  # exact  # noqa: E731
    rng = np.random.default_rng(1234)
    for trial in range(60):
        nkvh = int(rng.integers(1, 3))
        G = int(rng.integers(1, 4))
        nh = nkvh * G
        hd = int(rng.integers(1, 5))
        max_ctx = 8
        nkv = int(rng.integers(1, max_ctx + 1))
        q, k, v, pos = _case(1000 + trial, 1, nh, nkvh, hd, max_ctx, nkv)
        scale = float(np.float32(rng.uniform(0.1, 1.5)))
        got = oracle.decode_attn(q, k, v, pos, nkvh, scale, lib)
        kf = k.astype(np.float64)
        vf = v.astype(np.float64)
        for h in range(nh):
            g = h // G
            es = []
            for j in range(nkv):
                dot = sum((D(q[0, h, d]) * D(kf[0, j, g, d])
                           for d in range(hd)), decimal.Decimal(0))
                es.append(ctx.exp(ctx.multiply(D(np.float32(scale)), dot)))
            den = sum(es, decimal.Decimal(0))
            for d in range(hd):
                num = sum((e * D(vf[0, j, g, d]) for j, e in enumerate(es)),
                          decimal.Decimal(0))
                ref = float(ctx.divide(num, den))
                assert abs(got[0, h, d] - ref) <= 1e-13 * max(1.0, abs(ref)), (
                    trial, h, d, got[0, h, d], ref)


def pin_uniform_scores(lib):
    """Equal scores give the mean of V[0:nkv] (q = 0, scale = 0, equal K rows)."""
    B, nh, nkvh, hd, T = 2, 6, 2, 16, 40
    for nkv in (1, 7, 40):
        q, k, v, pos = _case(7, B, nh, nkvh, hd, T, nkv)
        mean = v[:, :nkv].astype(np.float64).mean(axis=1)       # [B][kv][hd]
        want = np.repeat(mean, nh // nkvh, axis=1)               # [B][nh][hd]
        _close(oracle.decode_attn(np.zeros_like(q), k, v, pos, nkvh, 0.3, lib),
               want, 1e-13, "q = 0")
        _close(oracle.decode_attn(q, k, v, pos, nkvh, 0.0, lib), want, 1e-13,
               "scale = 0")
        k_eq = np.broadcast_to(k[:, :1], k.shape).copy()
        _close(oracle.decode_attn(q, k_eq, v, pos, nkvh, 0.7, lib), want, 1e-13,
               "equal K rows")


def pin_two_rows_logistic(lib):
    """Two rows: o = V0 + sigma(s1 - s0)(V1 - V0), sigma via tanh."""
    hd, T = 4, 2
    for a, b, qs, scale in [(0.5, -1.25, 1.0, 1.0), (3.0, 2.0, 2.0, 0.25),
                            (-4.0, 26.0, 1.0, 1.0), (1.0, 1.0, 1.0, 1.0),
                            (0.0, -30.0, 0.5, 2.0)]:
        q = np.zeros((1, 1, hd), np.float32)
        q[0, 0, 0] = qs
        k = np.zeros((1, T, 1, hd), np.float16)
        k[0, 0, 0, 0] = a
        k[0, 1, 0, 0] = b
        k[0, :, 0, 1:] = 7.0    # ignored dims (q is zero there)
        v = np.array([[[[1.5, -2.0, 0.25, 8.0]], [[-0.5, 4.0, 0.25, -8.0]]]],
                     np.float16)
        pos = np.array([1], np.int32)
        x = float(np.float32(scale)) * qs * (b - a)
        sig = 0.5 * (1.0 + math.tanh(0.5 * x))
        v64 = v.astype(np.float64)[0, :, 0]
        want = v64[0] + sig * (v64[1] - v64[0])
        got = oracle.decode_attn(q, k, v, pos, 1, scale, lib)[0, 0]
        _close(got, want, 1e-14, f"two rows {a},{b}")


def pin_one_hot_dominant(lib):
    """A row scoring >= 70 above the rest returns that row's V (per group)."""
    B, nkvh, G, hd, T = 1, 3, 4, 64, 50
    nh = nkvh * G
    q, k, v, pos = _case(11, B, nh, nkvh, hd, T, T, q_scale=0.3)
    scale = 1.0 / 8.0
    star = [5, 17, 49]
    for g in range(nkvh):
        u = synth.offset_direction(q[0, g * G:(g + 1) * G], scale)
        k[0, star[g], g] = (k[0, star[g], g].astype(np.float64) + 80.0 * u
                            ).astype(np.float16)
    got = oracle.decode_attn(q, k, v, pos, nkvh, scale, lib)
    for h in range(nh):
        g = h // G
        _close(got[0, h], v[0, star[g], g].astype(np.float64), 1e-12,
               f"one-hot head {h}")


def pin_nkv_edges(lib):
    """nkv = 1 returns V[0] exactly; nkv = 0 returns 0; clamp past max_ctx."""
    B, nh, nkvh, hd, T = 3, 4, 2, 8, 6
    q, k, v, _ = _case(3, B, nh, nkvh, hd, T, 1)
    pos = np.array([0, -1, 2**31 - 1], np.int32)
    got = oracle.decode_attn(q, k, v, pos, nkvh, 0.35, lib)
    for h in range(nh):
        assert np.array_equal(got[0, h], v[0, 0, h // 2].astype(np.float64))
        assert np.array_equal(got[1, h], np.zeros(hd))
    full = oracle.decode_attn(q, k, v, np.array([0, -1, T - 1], np.int32),
                              nkvh, 0.35, lib)
    assert np.array_equal(got[2], full[2])


def pin_head_mapping(lib):
    """Query head h reads KV head h // G: equals a one-head call on that slice."""
    B, nkvh, G, hd, T = 2, 3, 2, 8, 12
    nh = nkvh * G
    q, k, v, pos = _case(21, B, nh, nkvh, hd, T, [12, 5])
    got = oracle.decode_attn(q, k, v, pos, nkvh, 0.4, lib)
    for h in range(nh):
        g = h // G
        one = oracle.decode_attn(q[:, h:h + 1].copy(),
                                 k[:, :, g:g + 1].copy(), v[:, :, g:g + 1].copy(),
                                 pos, 1, 0.4, lib)
        assert np.array_equal(got[:, h], one[:, 0]), h
    # perturbing KV head 1 moves exactly the heads of group 1
    k2 = k.copy()
    k2[:, :, 1] = -k2[:, :, 1]
    got2 = oracle.decode_attn(q, k2, v, pos, nkvh, 0.4, lib)
    for h in range(nh):
        same = np.array_equal(got2[:, h], got[:, h])
        assert same == (h // G != 1), h


def pin_permutation_invariance(lib):
    B, nh, nkvh, hd, T = 1, 4, 2, 16, 33
    q, k, v, pos = _case(31, B, nh, nkvh, hd, T, T)
    base = oracle.decode_attn(q, k, v, pos, nkvh, 0.25, lib)
    perm = np.random.default_rng(5).permutation(T)
    got = oracle.decode_attn(q, k[:, perm].copy(), v[:, perm].copy(), pos,
                             nkvh, 0.25, lib)
    _close(got, base, 1e-13, "row permutation")


def pin_linearity_in_v(lib):
    B, nh, nkvh, hd, T = 1, 4, 2, 8, 20
    q, k, _, pos = _case(41, B, nh, nkvh, hd, T, T)
    rng = np.random.default_rng(9)
    v1 = rng.integers(-8, 9, (B, T, nkvh, hd)).astype(np.float16)
    v2 = rng.integers(-8, 9, (B, T, nkvh, hd)).astype(np.float16)
    o1 = oracle.decode_attn(q, k, v1, pos, nkvh, 0.5, lib)
    o2 = oracle.decode_attn(q, k, v2, pos, nkvh, 0.5, lib)
    o12 = oracle.decode_attn(q, k, (v1 + v2).astype(np.float16), pos, nkvh, 0.5,
                             lib)
    _close(o12, o1 + o2, 1e-12, "V additivity")
    o_2 = oracle.decode_attn(q, k, (2 * v1).astype(np.float16), pos, nkvh, 0.5,
                             lib)
    assert np.array_equal(o_2, 2 * o1), "V scaling by 2"


def pin_convex_hull(lib):
    B, nh, nkvh, hd, T = 2, 6, 3, 16, 25
    q, k, v, pos = _case(51, B, nh, nkvh, hd, T, [25, 9], q_scale=3.0)
    got = oracle.decode_attn(q, k, v, pos, nkvh, 0.5, lib)
    nkv = [25, 9]
    for b in range(B):
        for h in range(nh):
            vv = v[b, :nkv[b], h // 2].astype(np.float64)
            assert np.all(got[b, h] >= vv.min(axis=0) - 1e-12)
            assert np.all(got[b, h] <= vv.max(axis=0) + 1e-12)


def pin_identical_heads(lib):
    B, nkvh, G, hd, T = 1, 2, 4, 16, 30
    q, k, v, pos = _case(61, B, nkvh * G, nkvh, hd, T, T)
    q[0, 1] = q[0, 0]
    q[0, 3] = q[0, 0]
    got = oracle.decode_attn(q, k, v, pos, nkvh, 0.25, lib)
    assert np.array_equal(got[0, 1], got[0, 0])
    assert np.array_equal(got[0, 3], got[0, 0])
    assert not np.array_equal(got[0, 2], got[0, 0])


def pin_split_combine_identity(lib):
    """R4 2.1: merging split records equals the unsplit softmax, any split."""
    for (B, nh, nkvh, hd, T, nkv, seed) in [(1, 4, 2, 16, 64, 64, 71),
                                           (2, 6, 2, 8, 100, [100, 37], 72),
                                           (1, 7, 1, 32, 40, 1, 73)]:
        q, k, v, pos = _case(seed, B, nh, nkvh, hd, T, nkv, q_scale=2.0)
        want = oracle.decode_attn(q, k, v, pos, nkvh, 0.5, lib)
        top = int(np.max(nkv))
        for S, blk in [(1, 0), (2, 0), (3, 0), (7, 0), (32, 0), (top, 0),
                       (top + 5, 0), (T, 1), (-(-T // 7), 7), (1, T), (3, 64)]:
            if blk and blk * S < T:
                continue
            rec = oracle.split_partials(q, k, v, pos, nkvh, 0.5, S, blk, lib)
            _close(oracle.combine(rec, lib), want, 1e-12, f"S={S} blk={blk}")


def pin_split_records(lib):
    """One-row splits hold (s_j, 1, V_j); idle splits hold (-inf, 0, 0)."""
    B, nh, nkvh, hd, T = 1, 4, 2, 8, 12
    nkv = 9
    q, k, v, pos = _case(81, B, nh, nkvh, hd, T, nkv)
    S = 12  # chunk = ceil(9/12) = 1 -> splits 9..11 idle
    rec = oracle.split_partials(q, k, v, pos, nkvh, 0.75, S, 0, lib)
    for sp in range(S):
        for h in range(nh):
            r = rec[0, sp, h]
            assert r[2] == sp and r[3] == min(nkv, sp + 1)
            if sp < nkv:
                s = 0.75 * float(np.dot(q[0, h].astype(np.float64),
                                        k[0, sp, h // 2].astype(np.float64)))
                assert abs(r[0] - s) <= 1e-14 * max(1.0, abs(s))
                assert r[1] == 1.0
                assert np.array_equal(r[4:], v[0, sp, h // 2].astype(np.float64))
            else:
                assert r[0] == -np.inf and r[1] == 0.0
                assert np.array_equal(r[4:], np.zeros(hd))


def pin_combine_worked(lib):
    """Hand-worked merges of R4 2.1's combine rule."""
    rec = np.zeros((1, 2, 1, 6))
    rec[0, 0, 0] = [0.0, 1.0, 0, 0, 2.0, 4.0]
    rec[0, 1, 0] = [math.log(2.0), 3.0, 0, 0, 1.0, 0.0]
    # gmx = ln 2, w = (1/2, 1): S = 3.5, acc = (2, 2) -> 4/7 each
    _close(oracle.combine(rec, lib)[0, 0], [4 / 7, 4 / 7], 1e-15, "worked")
    idle = np.zeros((1, 3, 1, 6))
    idle[0, :, 0, 0] = -np.inf
    assert np.array_equal(oracle.combine(idle, lib)[0, 0], [0.0, 0.0])
    one = idle.copy()
    one[0, 1, 0] = [5.0, 2.0, 0, 0, 3.0, -1.0]
    assert np.array_equal(oracle.combine(one, lib)[0, 0], [1.5, -0.5])


# --------------------------------------------------------------------------
# The cache append (#199 section 1) and several query rows (#199 section 2).
def _f16_bits_equal(ours, ref, what):
    """Bit equality of binary16 patterns; NaN patterns compare as NaN only."""
    ours = np.asarray(ours, np.uint16)
    ref = np.asarray(ref, np.uint16)
    nan_o = ((ours & 0x7C00) == 0x7C00) & ((ours & 0x03FF) != 0)
    nan_r = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x03FF) != 0)
    assert np.array_equal(nan_o, nan_r), f"{what}: NaN positions differ"
    bad = np.flatnonzero((ours != ref) & ~nan_r)
    assert bad.size == 0, (f"{what}: {bad.size} patterns differ, first "
                           f"ours {ours.flat[bad[0]]:#06x} ref {ref.flat[bad[0]]:#06x}")


def pin_f32_to_f16_numpy(lib):
    """binary32 -> binary16 equals numpy's conversion (an independent IEEE
    round-to-nearest-even implementation) on special values, values spread
    evenly over every exponent, and random bit patterns."""
    rng = np.random.default_rng(160)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.996,
                        65520.0, 65536.0, 1e9, 2.0**-24, 2.0**-25, 3 * 2.0**-26,
                        2.0**-14, 2.0**-14 - 2.0**-25, 1e-30, -1e-30, 1.0,
                        1.0 + 2.0**-11, 1.0 + 3 * 2.0**-11, 2049.0, 2051.0],
                       np.float32)
    spread = (rng.choice([-1.0, 1.0], 200_000) *
              np.exp2(rng.uniform(-30, 17, 200_000))).astype(np.float32)
    bits = rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)
    for name, x in (("special", special), ("spread", spread),
                    ("random bits", bits.view(np.float32))):
        with np.errstate(over="ignore", invalid="ignore"):
            ref = x.astype(np.float16).view(np.uint16)
        _f16_bits_equal(oracle.f32_to_f16(x, lib=lib), ref, name)


def pin_f32_to_f16_ties_and_round_trip(lib):
    """Every finite binary16 value converts back to itself; the midpoint of
    every pair of neighbours goes to the one with an even last bit (65520,
    between 65504 and the first value past the range, goes to infinity); one
    float32 step either side of a midpoint goes to the nearer neighbour."""
    h = np.arange(0, 0x7C00, dtype=np.uint16)          # +0 .. 65504
    vals = h.view(np.float16).astype(np.float32)
    for sign in (0, 0x8000):
        s = -1.0 if sign else 1.0
        _f16_bits_equal(oracle.f32_to_f16(s * vals, lib=lib), h | sign,
                        "round trip")
        a = h.view(np.float16).astype(np.float64)
        b = np.append(a[1:], 65536.0)                     # next value up
        mid = ((a + b) / 2).astype(np.float32)            # exact in float32
        assert np.array_equal(mid.astype(np.float64), (a + b) / 2)
        nxt = np.append(h[1:], np.uint16(0x7C00))
        even = np.where(h % 2 == 0, h, nxt).astype(np.uint16)
        _f16_bits_equal(oracle.f32_to_f16(s * mid, lib=lib), even | sign, "ties")
        up = np.nextafter(mid, np.float32(np.inf))
        dn = np.nextafter(mid, np.float32(0))
        _f16_bits_equal(oracle.f32_to_f16(s * up, lib=lib), nxt | sign, "above")
        _f16_bits_equal(oracle.f32_to_f16(s * dn, lib=lib), h | sign, "below")


def pin_append_kv(lib):
    """Appending writes the fp16 of each new row at positions[b] - (n-1) + t
    and nothing else; rows outside [0, max_ctx) are dropped. The expected
    caches are built with numpy indexing and numpy's conversion."""
    rng = np.random.default_rng(161)
    B, nkvh, hd, T = 4, 2, 4, 8
    for n_rows in (1, 3):
        kc = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
        vc = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
        kn = (rng.standard_normal((B, n_rows, nkvh, hd)) * 300).astype(np.float32)
        vn = rng.standard_normal((B, n_rows, nkvh, hd)).astype(np.float32)
        kn[0, 0, 0, :4] = [np.nan, np.inf, 1e-7, 7e4]
        pos = np.array([n_rows - 1, T - 1, T + 1, 1], np.int32)
        ek = kc.view(np.uint16).copy()
        ev = vc.view(np.uint16).copy()
        for b in range(B):
            for t in range(n_rows):
                p = int(pos[b]) - (n_rows - 1) + t
                if 0 <= p < T:
                    with np.errstate(over="ignore", invalid="ignore"):
                        ek[b, p] = kn[b, t].astype(np.float16).view(np.uint16)
                        ev[b, p] = vn[b, t].astype(np.float16).view(np.uint16)
        k2, v2 = oracle.append_kv(kn, vn, kc, vc, pos, lib=lib)
        _f16_bits_equal(k2, ek, f"append K, {n_rows} rows")
        _f16_bits_equal(v2, ev, f"append V, {n_rows} rows")


def _causal_reference(q, k, v, pos, scale):
    """Textbook masked attention in matrix form (numpy, double): for sequence
    b, head h, S = Q Kᵀ scale over the whole cache, entries j > (row
    position) set to -inf, row softmax, times V; a row with no keys is 0."""
    B, n_q, nh, hd = q.shape
    T, nkvh = k.shape[1], k.shape[2]
    G = nh // nkvh
    out = np.zeros((B, n_q, nh, hd))
    for b in range(B):
        rowpos = int(pos[b]) - (n_q - 1) + np.arange(n_q)
        mask = np.arange(T)[None, :] > rowpos[:, None]
        for h in range(nh):
            Kf = k[b, :, h // G, :].astype(np.float64)
            Vf = v[b, :, h // G, :].astype(np.float64)
            S = q[b, :, h, :].astype(np.float64) @ Kf.T * float(np.float32(scale))
            S[mask] = -np.inf
            for t in range(n_q):
                if not np.isfinite(S[t]).any():
                    continue
                w = np.exp(S[t] - S[t].max())
                out[b, t, h] = (w @ Vf) / w.sum()
    return out


def pin_rows_causal(lib):
    """Several query rows equal textbook causal attention: a prefill from
    empty (rows at 0..n-1), a chunk after a cached prefix, a chunk whose
    first rows sit before position 0 (no keys: output 0), and one single-row
    decode."""
    rng = np.random.default_rng(162)
    B, nh, nkvh, hd, T = 4, 4, 2, 8, 12
    for n_q in (1, 4):
        q = rng.standard_normal((B, n_q, nh, hd)).astype(np.float32)
        k = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
        v = rng.standard_normal((B, T, nkvh, hd)).astype(np.float16)
        pos = np.array([n_q - 1, 9, 1, T - 1], np.int32)
        scale = 0.35
        got = oracle.decode_attn_rows(q, k, v, pos, nkvh, scale, lib=lib)
        _close(got, _causal_reference(q, k, v, pos, scale), 1e-12,
               f"causal rows n_q={n_q}")
    # a chunk that fills the cache: every row sees exactly its prefix
    q = rng.standard_normal((1, T, nh, hd)).astype(np.float32)
    k = rng.standard_normal((1, T, nkvh, hd)).astype(np.float16)
    v = rng.standard_normal((1, T, nkvh, hd)).astype(np.float16)
    pos = np.array([T - 1], np.int32)
    got = oracle.decode_attn_rows(q, k, v, pos, nkvh, 0.2, lib=lib)
    _close(got, _causal_reference(q, k, v, pos, 0.2), 1e-12, "full prefill")
    # row 0 of that prefill sees only key 0: exactly V[0]
    G = nh // nkvh
    for h in range(nh):
        assert np.array_equal(got[0, 0, h], v[0, 0, h // G].astype(np.float64))
