"""CPU pins of the lane decoder's comparison plans.

"LazyWeights", section "3 . Decode on demand": a lane finds a code's length
by comparing the next 11 stream bits with one limit per length.  The GPU
kernels do this with sums of absolute differences over bytes gathered from
the peek (lane_decode.hpp); the bundle builder derives, per table, which
bytes to gather and which thresholds to compare (the plan stored with the
derived GPU tables).

These tests take the plan a bundle carries and evaluate, on the CPU, the
instruction sequence the kernels issue (v_perm_b32, v_add_u32 and v_sub_u32
with clamp, v_sad_u8, v_sad_u16, written here from their instruction-set
definitions)
for every 11-bit peek followed by arbitrary stream bits.  The result must
equal the length the canonical table defines (the first length whose limit
exceeds the peek), on the workloads' tables and on random complete codes that
reach every plan.  No GPU call is made.
"""
import numpy as np
import pytest

import decode_gemv_amd as dg
import synth
from support import codes_over, plan_of, random_complete_lengths

PBASE, CSEL, SBASE = 1024, 0xD07, 526
PLANS = {0: "compact", 1: "r2", 2: "r2k", 3: "r2x2", 4: "gen", 5: "s2k"}
M32 = 0xFFFFFFFF


# ------------------------------------------------------------ instruction models

def v_perm_b32(s0, s1, sel):
    """Byte i of the result is chosen by byte i of sel from the eight bytes of
    {s0, s1} (s1 the low word); 12 gives 0x00, 13 and above 0xFF."""
    src = (np.uint64(s0) << np.uint64(32)) | np.uint64(s1)
    out = np.zeros_like(np.asarray(s1, dtype=np.uint64))
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        assert b < 8 or b >= 12, "sign-replicating selectors are not used"
        if b < 8:
            v = (src >> np.uint64(8 * b)) & np.uint64(0xFF)
        elif b == 12:
            v = np.zeros_like(out)
        else:
            v = np.full_like(out, 0xFF)
        out |= v << np.uint64(8 * i)
    return out


def v_sad_u8(a, b, c):
    a = np.asarray(a, np.int64)
    r = np.asarray(c, np.int64).copy()
    for i in range(4):
        r += np.abs(((a >> (8 * i)) & 0xFF) - ((b >> (8 * i)) & 0xFF))
    return r & M32


def v_sad_u16(a, b, c):
    a = np.asarray(a, np.int64)
    r = np.asarray(c, np.int64).copy()
    for i in range(2):
        r += np.abs(((a >> (16 * i)) & 0xFFFF) - ((b >> (16 * i)) & 0xFFFF))
    return r & M32


def v_add_u32_clamp(a, b):
    return np.minimum(np.asarray(a, np.int64) + int(b), M32)


def v_sub_u32_clamp(a, b):
    return np.maximum(np.asarray(a, np.int64) - int(b), 0)


# ------------------------------------------------------------ the stored plan

def kernel_count(pl, hi):
    """A = s2 - s1 as the kernels compute it for peek registers hi."""
    P = pl["plan"]
    s1 = np.zeros(hi.shape, np.int64)
    s2 = np.full(hi.shape, pl["sad_k"], np.int64)
    if P in (0, 4):
        p8 = v_perm_b32(hi, hi, 0x03030303)
        if P == 4:
            p16 = v_perm_b32(hi, hi, 0x03020302)
            s1 = v_sad_u16(p16, pl["c16m1"], s1)
            s2 = v_sad_u16(p16, pl["c16"], s2)
            s1 = v_sad_u8(p8, pl["c8m1"][1], s1)
            s2 = v_sad_u8(p8, pl["c8"][1], s2)
        s1 = v_sad_u8(p8, pl["c8m1"][0], s1)
        s2 = v_sad_u8(p8, pl["c8"][0], s2)
    else:
        if P == 1:
            x1 = v_perm_b32(hi, hi, 0x03030303)
        elif P == 5:
            x1 = v_perm_b32(v_sub_u32_clamp(hi, pl["xk"][0]), hi, pl["xsel"][0])
        else:
            x1 = v_perm_b32(v_add_u32_clamp(hi, pl["xk"][0]), hi, pl["xsel"][0])
        x2 = v_perm_b32(v_add_u32_clamp(hi, pl["xk"][1]), hi, pl["xsel"][1]) if P == 3 else x1
        s1 = v_sad_u8(x1, pl["c8m1"][0], s1)
        s2 = v_sad_u8(x1, pl["c8"][0], s2)
        s1 = v_sad_u8(x2, pl["c8m1"][1], s1)
        s2 = v_sad_u8(x2, pl["c8"][1], s2)
    return (s2 - s1) & M32


def table_of(bundle):
    t = dg.lw_bundle_region(bundle, dg.LW_REG_TABLE, np.uint16)
    return dict(count=t[0:12].astype(np.int64), limit=t[24:36].astype(np.int64))


def check_bundle(bundle, rng, junk_draws=3):
    """Every valid peek, several random tails: the plan's count gives the
    canonical length (and, for compact tables, the shift byte -len)."""
    info = dg.lw_bundle_get_info(bundle)
    t = table_of(bundle)
    pl = plan_of(bundle)
    lmin, lmax = info["min_len"], info["max_len"]
    end = int(t["limit"][lmax])                      # peeks past the last limit never occur
    p = np.arange(end, dtype=np.int64)
    want = np.full(end, lmax, np.int64)
    for L in range(lmax - 1, lmin - 1, -1):
        want[p < t["limit"][L]] = L
    for d in range(junk_draws):
        junk = {0: np.zeros(end, np.int64), 1: np.full(end, (1 << 21) - 1, np.int64)}.get(
            d, rng.integers(0, 1 << 21, end, dtype=np.int64))
        hi = (p << 21) | junk
        A = kernel_count(pl, hi)
        if pl["plan"] == 0:
            used = [L for L in range(1, 12) if t["count"][L]]
            r = (CSEL - A) // 2
            assert np.array_equal(A, CSEL - 2 * r)
            got = np.array(used)[r]
            # the shift byte the perm table gives is -len mod 256, upper bytes 0xFF
            lut = (pl["lut_hi"] << 32) | pl["lut_lo"]
            s = v_perm_b32(pl["lut_hi"], pl["lut_lo"], int(A[0]))
            for i in range(0, end, max(1, end // 64)):
                s = int(v_perm_b32(pl["lut_hi"], pl["lut_lo"], int(A[i])))
                assert s == (-int(got[i])) & M32, (i, hex(s), got[i], hex(lut))
        elif pl["plan"] == 5:
            # sparse: the count r of used-length limits passed, A = SBASE - 2r;
            # the low byte of the shift perm(lut, A >> 1) is -len mod 256
            used = [L for L in range(1, 12) if t["count"][L]]
            r = (SBASE - A) // 2
            assert np.array_equal(A, SBASE - 2 * r) and r.min() >= 0 and r.max() < len(used)
            got = np.array(used)[r]
            for i in range(0, end, max(1, end // 64)):
                sh = int(v_perm_b32(pl["lut_hi"], pl["lut_lo"], int(A[i]) >> 1))
                assert sh & 0xFF == (-int(got[i])) & 0xFF, (i, hex(sh), got[i])
        else:
            assert np.all((PBASE - A) % 2 == 0)
            got = (PBASE - A) // 2
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (PLANS[pl["plan"]], bad[:5], got[bad[:5]], want[bad[:5]])
    return pl["plan"]


def test_plans_of_workload_tables():
    rng = np.random.default_rng(7)
    seen = {}
    for wl in ("q4_256x1024", "q4_up_14336x4096", "q4_down_4096x14336", "q6_mlp_70b"):
        mat = synth.WORKLOADS[wl][0]
        kind = dg.LW_Q4_PAIR if mat.kind == "q4" else dg.LW_Q6_SINGLE
        codes, d, m, _ = synth.gen_q(mat, rows=min(mat.rows, 512), cols=min(mat.cols, 4096))
        for build in (dg.lw_bundle_build_q, dg.lw_bundle_build_q_compact):
            seen[(wl, build.__name__)] = PLANS[check_bundle(build(kind, codes, d, m), rng)]
    w, _ = synth.gen_bf16(synth.WORKLOADS["bf16_up_14336x4096"][0], rows=256, cols=4096)
    seen["bf16"] = PLANS[check_bundle(dg.lw_bundle_build_bf16(w), rng)]
    # the optimal codes of the 4-bit and 6-bit workloads take the residue plans
    assert seen[("q4_up_14336x4096", "lw_bundle_build_q")] in ("r2k", "r2x2", "r2")
    assert seen[("q6_mlp_70b", "lw_bundle_build_q")] in ("r2k", "r2x2", "r2")
    assert seen[("q4_up_14336x4096", "lw_bundle_build_q_compact")] == "compact"
    # the bf16 exponent table (lengths 2..7, 9, 11) compares its used lengths only
    assert seen["bf16"] == "s2k"


def test_sparse_group_shift_sum():
    """The sparse plan's shifts carry other table bytes above their low byte;
    a group's four shifts summed, low byte sign-extended, is -sum(len), and
    each shift's low five bits are 32 - len (what the decoder relies on)."""
    w, _ = synth.gen_bf16(synth.WORKLOADS["bf16_up_14336x4096"][0], rows=128, cols=1024)
    b = dg.lw_bundle_build_bf16(w)
    pl, t = plan_of(b), table_of(b)
    assert pl["plan"] == 5
    used = [L for L in range(1, 12) if t["count"][L]]
    n = len(used)
    shift = [int(v_perm_b32(pl["lut_hi"], pl["lut_lo"], (SBASE - 2 * r) >> 1)) for r in range(n)]
    for r in range(n):
        assert shift[r] & 31 == (32 - used[r]) & 31
    for r0 in range(n):
        for r1 in range(n):
            for r2 in range(n):
                for r3 in range(n):
                    tt = (shift[r0] + shift[r1] + shift[r2] + shift[r3]) & M32
                    low = tt & 0xFF
                    sext = low - 256 if low >= 128 else low
                    assert sext == -(used[r0] + used[r1] + used[r2] + used[r3])


@pytest.mark.parametrize("seed", range(6))
def test_plans_of_random_complete_codes(seed):
    """Random complete codes with 2..256 symbols and lengths up to 11: every
    plan the builder picks counts every peek right."""
    rng = np.random.default_rng(1000 + seed)
    seen = set()
    for trial in range(40):
        kind = dg.LW_Q4_PAIR if trial % 3 else dg.LW_Q6_SINGLE
        n_alpha = 256 if kind == dg.LW_Q4_PAIR else 64
        n_sym = int(rng.integers(2, n_alpha + 1))
        depth = int(rng.integers(max(1, int(np.ceil(np.log2(n_sym)))), 12))
        lens, syms = random_complete_lengths(rng, n_alpha, n_sym, depth)
        codes = codes_over(rng, kind == dg.LW_Q4_PAIR, syms)
        d = np.zeros((64, 1), np.uint16)
        b = dg.lw_bundle_build_q_lens(kind, codes, d, d, lens)
        seen.add(PLANS[check_bundle(b, rng, junk_draws=2)])
    assert seen, "no table checked"


def test_every_plan_is_reached():
    """The random tables of the test above and the bf16 workload's table
    reach all six plans, so each plan's arithmetic is pinned."""
    rng = np.random.default_rng(99)
    w, _ = synth.gen_bf16(synth.WORKLOADS["bf16_up_14336x4096"][0], rows=64, cols=256)
    seen = {PLANS[check_bundle(dg.lw_bundle_build_bf16(w), rng, junk_draws=2)]}
    for trial in range(300):
        kind = dg.LW_Q4_PAIR
        n_sym = int(rng.integers(2, 257))
        depth = int(rng.integers(max(1, int(np.ceil(np.log2(n_sym)))), 12))
        lens, syms = random_complete_lengths(rng, 256, n_sym, depth)
        b = dg.lw_bundle_build_q_lens(kind, codes_over(rng, True, syms), np.zeros((64, 1), np.uint16),
                                      np.zeros((64, 1), np.uint16), lens)
        pl = plan_of(b)["plan"]
        if PLANS[pl] not in seen:
            check_bundle(b, rng, junk_draws=2)
            seen.add(PLANS[pl])
        if len(seen) == len(PLANS):
            break
    assert seen == set(PLANS.values()), seen


def test_corrupt_plan_rejected():
    """A loaded image whose stored plan disagrees with its table is refused."""
    codes, d, m, _ = synth.gen_q_custom(64, 256, 5)
    b = dg.lw_bundle_build_q(dg.LW_Q4_PAIR, codes, d, m)
    img = dg.lw_bundle_image(b).copy()
    info = dg.lw_bundle_get_info(b)
    off = info["region_offset"][dg.LW_REG_GPUTAB] + 4 * (16 * 3 + 256 * 3) + 8   # c8[0]
    img[off] ^= 1
    with pytest.raises(dg.LwError) as e:
        dg.lw_bundle_load(img)
    assert e.value.status == dg.LW_E_FORMAT
