"""Page-balanced keys: the active reading of variance normalisation (CPU, oracle).

The pages name variance normalisation as a pipeline stage without a formula
(dothoosh.com, "KVarN vs TurboQuant: 5x more context with higher accuracy",
the four-stage list, stage 2; the Persian text reads it as an iterative
normalisation, and the closing paragraph credits the method with removing
fluctuations in logarithmic space).  The v1 format divides each token group
by its RMS, which leaves the codes unchanged in exact arithmetic.  The
page-balanced reading iterates column and row second moments over a page of
one KV head and keeps every scale a power of two (kvqo_block_variant).

Pins, none of which re-types the oracle's formulas:
  * three hand-derived blocks (tests/golden/page_balance_*.txt): exponents
    at 1, 2 and 3 passes (the pass order and count), codes, fp16 metadata,
    the floor for zero columns and the stored byte of each scale;
  * zero passes is the per-token encoder, bit for bit;
  * the scaled rows are quantised by the encoder: error within s/2 per
    element in the scaled domain, nearest level by brute force;
  * scale equivariance of the whole block (powers of two);
  * absent rows are zeros in the sums: a block with holes equals the block
    of its present rows;
  * the append writes the v1 layout plus the scale bytes, values unchanged;
  * decode over a page-balanced cache whose scales are all 1 equals the v1
    decode of the same bytes (itself pinned to SDPA in test_oracle).
"""
import math
import os

import numpy as np
import pytest

import oracle

D = 128
SCALE = 1.0 / math.sqrt(D)
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
H = np.array([[1]])
while H.shape[0] < D:
    H = np.block([[H, H], [H, -H]])


def _fixture(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = [s.strip() for s in line.split("=", 1)]
                out[k] = v
    return out


def _ints(v):
    return [int(t, 0) for t in v.split()]


LO, HI = np.arange(D) < 64, np.arange(D) >= 64


def test_hand_derived_two_token_block():
    f = _fixture("page_balance_two_tokens.txt")
    x = np.zeros((2, D), np.float16)
    x[0, int(f["x0_channel"])] = 1
    for ch, val in zip(_ints(f["x1_channels"]), f["x1_values"].split()):
        x[1, ch] = float(val)
    for iters in (1, 2, 3):
        codes, rec, s, z, e = oracle.block_variant(x, 4, iters)
        assert np.all(e[LO] == int(f[f"iters{iters}_exp_lo"])) and np.all(e[HI] == int(f[f"iters{iters}_exp_hi"]))
    codes, rec, s, z, e = oracle.block_variant(x, 4, 2)
    h3, h5 = H[:, 3], H[:, 5]
    for t, h in ((0, h3), (1, h5)):
        for part, mask in (("lo", LO), ("hi", HI)):
            plus, minus = _ints(f[f"t{t}_{part}_codes"])
            assert np.all(codes[t][mask & (h > 0)] == plus) and np.all(codes[t][mask & (h < 0)] == minus)
        assert s[t] == int(f[f"t{t}_s"], 16) and z[t] == int(f[f"t{t}_z"], 16)
    # the stored byte of each scale (the page-balanced append writes it)
    pool = np.zeros((1, 1, oracle.PB_REGION), np.uint8)
    v = np.zeros((2, 1, D), np.float16)
    assert oracle.quantize_append_pb(x[:, None, :], v, np.array([0, 1]), pool) == 0
    scale_bytes = pool[0, 0, 1664:]
    assert np.all(scale_bytes[LO] == int(f["byte_exp_lo"], 16)) and np.all(scale_bytes[HI] == int(f["byte_exp_hi"], 16))
    # the slot dequantisation reads the stored bytes back to the hand-derived
    # values: 2^e (s c + z) with the fixture's codes, s, z and exponents
    hs = [oracle.half_to_double(int(f[f"t{t}_s"], 16)) for t in range(2)]
    hz = [oracle.half_to_double(int(f[f"t{t}_z"], 16)) for t in range(2)]
    e_hand = np.where(LO, int(f["iters2_exp_lo"]), int(f["iters2_exp_hi"]))
    for t, h in ((0, h3), (1, h5)):
        c_hand = np.zeros(D)
        for part, mask in (("lo", LO), ("hi", HI)):
            plus, minus = _ints(f[f"t{t}_{part}_codes"])
            c_hand[mask] = np.where(h[mask] > 0, plus, minus)
        k_slot, _ = oracle.dequant_slot_pb(np.ascontiguousarray(pool[0, 0]), t)
        assert np.array_equal(k_slot, H @ np.ldexp(hs[t] * c_hand + hz[t], e_hand) / 128.0)
    # the rebuilt block: 2^e (s c + z), un-rotated
    y = np.ldexp(np.array([oracle.half_to_double(int(s[t])) for t in range(2)])[:, None] * codes +
                 np.array([oracle.half_to_double(int(z[t])) for t in range(2)])[:, None], e[None, :])
    assert np.array_equal(rec, y @ H / 128.0)


def test_hand_derived_separable_page():
    f = _fixture("page_balance_separable.txt")
    x = np.zeros((16, D), np.float16)
    for t in range(16):
        a, k = (1, 2)[t % 2], t + 1
        x[t, k] = 2.5 * a
        x[t, k + 64] = -1.5 * a
    for iters in (1, 2, 3):
        codes, rec, s, z, e = oracle.block_variant(x, 4, iters)
        assert np.all(e[LO] == int(f["exp_lo"])) and np.all(e[HI] == int(f["exp_hi"]))
        for t in range(16):
            h = H[:, t + 1]
            assert np.all(codes[t][h > 0] == int(f["codes_plus"])) and np.all(codes[t][h < 0] == int(f["codes_minus"]))
            a = "a1" if t % 2 == 0 else "a2"
            assert s[t] == int(f["s_" + a], 16) and z[t] == int(f["z_" + a], 16)
    pool = np.zeros((1, 1, oracle.PB_REGION), np.uint8)
    assert oracle.quantize_append_pb(x[:, None, :], np.zeros((16, 1, D), np.float16), np.arange(16), pool) == 0
    b = pool[0, 0, 1664:]
    assert np.all(b[LO] == int(f["byte_lo"], 16)) and np.all(b[HI] == int(f["byte_hi"], 16))


def test_hand_derived_zero_columns_take_the_floor():
    f = _fixture("page_balance_zero_columns.txt")
    x = np.zeros((1, D), np.float16)
    x[0, 0] = x[0, 1] = 1
    even = np.arange(D) % 2 == 0
    for iters in (1, 2):
        codes, rec, s, z, e = oracle.block_variant(x, 4, iters)
        assert np.all(e[even] == int(f["exp_even"])) and np.all(e[~even] == int(f["exp_odd"]))
        assert np.all(codes[0][even] == int(f["codes_even"])) and np.all(codes[0][~even] == int(f["codes_odd"]))
        assert s[0] == int(f["s"], 16) and z[0] == int(f["z"], 16)
        y = np.where(even, float(f["rec_even"]), 0.0)
        assert np.array_equal(rec[0], H @ y / 128.0)
    pool = np.zeros((1, 1, oracle.PB_REGION), np.uint8)
    assert oracle.quantize_append_pb(x[:, None, :], np.zeros((1, 1, D), np.float16), np.array([0]), pool) == 0
    b = pool[0, 0, 1664:]
    assert np.all(b[even] == int(f["byte_even"], 16)) and np.all(b[~even] == int(f["byte_odd"], 16))


def test_region_size():
    """1664 bytes of the K4V2 region plus one scale byte per rotated channel:
    112 bytes per token and KV head (8 more than K4V2, 24 fewer than k4v4)."""
    assert oracle.pb_region_bytes() == oracle.PB_REGION == 1664 + 128
    assert oracle.PB_REGION % 128 == 0 and oracle.PB_REGION // 16 == 112


def test_zero_passes_is_the_per_token_encoder():
    """iters = 0: the same codes and metadata as the group encoder (keys' zero
    offset) and the same reconstruction s c + z, un-rotated."""
    rng = np.random.default_rng(1)
    for bits in (4, 2, 8):
        x = (rng.standard_normal((16, D)) * [0.01, 1, 30][bits % 3]).astype(np.float16)
        codes, rec, s, z, e = oracle.block_variant(x, bits, 0)
        assert np.all(e == 0)
        for t in range(16):
            c, s1, z1 = oracle.quantize_group(x[t], bits, offset_mode=0)
            assert np.array_equal(codes[t], c) and s[t] == s1 and z[t] == z1
            y = oracle.half_to_double(s1) * c.astype(np.float64) + oracle.half_to_double(z1)
            assert np.max(np.abs(rec[t] - H @ y / 128)) < 1e-12


@pytest.mark.parametrize("bits", [4, 2])
def test_scaled_rows_error_bound_and_nearest_level(bits):
    """In the scaled domain Yhat = Y 2^-e (Y the exact rotation), every element
    is within s/2 (plus fp16 slack) of its level s c + z, which is the nearest
    of the row's levels: the rows go through the encoder's RTN."""
    rng = np.random.default_rng(7 + bits)
    L = (1 << bits) - 1
    levels = np.arange(L + 1, dtype=np.float64)
    for trial in range(40):
        # loud and quiet rotated-domain channels (the rotation would even out
        # original-domain ones), taken back to the original domain
        y = rng.standard_normal((16, D)) * rng.choice([0.05, 1, 20], D)
        x16 = (y @ H / 128.0).astype(np.float16)
        codes, rec, s, z, e = oracle.block_variant(x16, bits, 2)
        assert e.max() <= 6 and e.min() >= -6 and (e != 0).any()
        Y = x16.astype(np.float64) @ H          # rows: H x (H symmetric)
        Yh = Y * 2.0 ** -e.astype(np.float64)
        for t in range(16):
            sv, zv = oracle.half_to_double(int(s[t])), oracle.half_to_double(int(z[t]))
            lev = sv * codes[t] + zv
            slack = 2.0 ** -10 * (L * sv + abs(zv)) + 1e-6 * np.abs(Yh[t]).max()
            err = np.abs(Yh[t] - lev)
            assert np.all(err <= sv / 2 + slack)
            best = np.min(np.abs(Yh[t][:, None] - (sv * levels[None, :] + zv)), axis=1)
            assert np.all(err <= best + slack)


def test_power_of_two_scale_equivariance_of_the_block():
    """Scaling the whole block by 2^k leaves codes and exponents unchanged
    and scales s and z by exactly 2^k (every sum scales by 2^2k, so each
    exponent moves by k before it is taken relative to the loudest)."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        # magnitudes in [0.01, 4] times a per-channel factor in [0.2, 3]:
        # every scaled copy stays a normal fp16
        x16 = (rng.choice([-1, 1], (16, D)) * rng.uniform(0.01, 4, (16, D)) * rng.uniform(0.2, 3, D)).astype(np.float16)
        c0, _, s0, z0, e0 = oracle.block_variant(x16, 4, 2)
        for k in (-2, 3):
            xk = (x16.astype(np.float64) * 2.0 ** k).astype(np.float16)
            assert np.array_equal(xk.astype(np.float64), x16.astype(np.float64) * 2.0 ** k)
            ck, _, sk, zk, ek = oracle.block_variant(xk, 4, 2)
            assert np.array_equal(ck, c0) and np.array_equal(ek, e0)
            for t in range(16):
                assert oracle.half_to_double(int(sk[t])) == oracle.half_to_double(int(s0[t])) * 2.0 ** k
                assert oracle.half_to_double(int(zk[t])) == oracle.half_to_double(int(z0[t])) * 2.0 ** k


def test_absent_rows_are_zeros():
    """A block with absent rows gives its present rows the codes, metadata
    and exponents of the block made of those rows alone (zeros add exactly
    in the fixed-tree sums, wherever they sit)."""
    rng = np.random.default_rng(12)
    x16 = rng.standard_normal((13, D)).astype(np.float16)
    present = np.array([1, 0, 1, 1, 0, 0, 1, 1, 1, 0, 1, 1, 0], bool)
    c, _, s, z, e = oracle.block_variant(x16, 4, 2, present=present)
    c2, _, s2, z2, e2 = oracle.block_variant(x16[present], 4, 2)
    assert np.array_equal(e, e2)
    assert np.array_equal(c[present], c2) and np.array_equal(s[present], s2) and np.array_equal(z[present], z2)


def test_append_pb_layout_and_values():
    """Whole-page append: page base/16 from slot 0; keys = the block variant's
    codes and metadata in the K4V2 key layout, one scale byte per channel after
    the region; values = the v1 encoder's groups; tokens breaking the slot run
    and blocks starting off a page boundary are not written."""
    rng = np.random.default_rng(13)
    T, Hh = 40, 2
    k = rng.standard_normal((T, Hh, D)).astype(np.float16)
    v = rng.standard_normal((T, Hh, D)).astype(np.float16)
    slots = np.array([16 * 3 + r for r in range(16)] + [16 * 1 + r for r in range(16)] + [16 * 0 + r for r in range(8)])
    slots[20] = -1            # a hole in page 1
    slots[33] = 5             # breaks the run of page 0 (base 0): not written
    pool = np.full((5, Hh, oracle.PB_REGION), 0xAB, np.uint8)
    assert oracle.quantize_append_pb(k, v, slots, pool) == 0
    for page, first, n in ((3, 0, 16), (1, 16, 16), (0, 32, 8)):
        present = np.array([slots[first + r] == 16 * page + r for r in range(n)])
        for h in range(Hh):
            region = pool[page, h]
            kc, _, ks, kz, e = oracle.block_variant(k[first:first + n, h], 4, oracle.pb_iters(), present=present)
            assert np.array_equal(region[1664:], ((e + 15) * 4).astype(np.uint8))
            for r in range(16):
                if r < n and present[r]:
                    lk = oracle.load_token(region[:1664].copy(), r)
                    vc, vs, vmu = oracle.quantize_group(v[first + r, h], 2)
                    assert np.array_equal(lk[0], kc[r]) and lk[1] == ks[r] and lk[2] == kz[r]
                    assert np.array_equal(lk[3], vc) and lk[4] == vs and lk[5] == vmu
                else:        # untouched slot: canary bytes remain
                    assert np.all(region[64 * r:64 * r + 64] == 0xAB)
    assert np.all(pool[2] == 0xAB) and np.all(pool[4] == 0xAB)
    # a block whose first slot is not a page boundary, or beyond the pool
    pool2 = np.zeros((2, 1, oracle.PB_REGION), np.uint8)
    assert oracle.quantize_append_pb(k[:16, :1], v[:16, :1], np.arange(3, 19), pool2) == 0
    assert not pool2.any()
    assert oracle.quantize_append_pb(k[:16, :1], v[:16, :1], np.arange(32, 48), pool2) == -1


def test_decode_pb_with_unit_scales_is_the_v1_decode():
    """A page-balanced cache whose scale bytes all encode 2^0 decodes exactly
    as the v1 decode of its 1664-byte prefix (pinned to SDPA on on-grid
    caches in test_oracle); a scale of 2^e multiplies that channel of every
    key by 2^e."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, n = 2, 4, 2, 37
    pages = 2 * 3
    pool = np.zeros((pages, Hkv, oracle.PB_REGION), np.uint8)
    bt = rng.permutation(pages).astype(np.int32).reshape(B, 3)
    for b in range(B):
        kk = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        vv = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        t = np.arange(n)
        oracle.quantize_append_pb(kk, vv, bt[b, t // 16].astype(np.int64) * 16 + t % 16, pool)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    lens = np.array([n, 21])
    unit = pool.copy()
    unit[:, :, 1664:] = 0x3C
    a = oracle.decode_attention_pb(unit, bt, lens, q, SCALE)
    b1 = oracle.decode_attention(np.ascontiguousarray(unit[:, :, :1664]), bt, lens, q, SCALE)
    assert np.array_equal(a, b1)
    # one channel scaled by 2^-3: every dequantised rotated key of that channel scales
    scaled = unit.copy()
    scaled[:, :, 1664 + 17] = (-3 + 15) * 4
    for p in range(pages):
        for h in range(Hkv):
            for r in range(16):
                k0, v0 = oracle.dequant_slot_pb(np.ascontiguousarray(unit[p, h]), r)
                k1, v1 = oracle.dequant_slot_pb(np.ascontiguousarray(scaled[p, h]), r)
                yk0, yk1 = H @ k0, H @ k1          # back to the rotated domain (x128)
                assert np.allclose(yk1[17], yk0[17] / 8, atol=1e-9) and np.allclose(np.delete(yk1, 17), np.delete(yk0, 17), atol=1e-9)
                assert np.array_equal(v0, v1)
    # the real exponents change the result, and it stays close to the fp16 attention
    real = oracle.decode_attention_pb(pool, bt, lens, q, SCALE)
    assert not np.array_equal(real, a)


def _blocks(kind, n, rng, T=16):
    out = []
    for _ in range(n):
        if kind == "normal":
            x = rng.standard_normal((T, D))
        elif kind == "outlier_channels":          # 3 channels x15, as the decode workloads' keys
            x = rng.standard_normal((T, D))
            x[:, [5, 40, 77]] *= 15
        elif kind == "student_t3":
            x = rng.standard_t(3, (T, D))
        elif kind == "channel_offsets":           # a per-channel mean shared by the page's tokens
            x = rng.standard_normal((T, D)) + 3 * rng.standard_normal(D)
        elif kind == "rotated_column":            # one rotated-domain channel x64
            y = rng.standard_normal((T, D))
            y[:, 9] *= 64
            x = y @ H / 128 * np.sqrt(D)
        out.append(x.astype(np.float16))
    return out


def _rel_mse(blocks, bits, iters):
    err = tot = 0.0
    for x in blocks:
        rec = oracle.block_variant(x, bits, iters)[1]
        xd = x.astype(np.float64)
        err += np.sum((rec - xd) ** 2)
        tot += np.sum(xd ** 2)
    return err / tot


def test_column_balancing_absorbs_a_loud_rotated_channel():
    """One rotated-domain channel 64x louder than the rest sets every token's
    range for per-token RTN; balancing gives it its own power-of-two scale,
    so the error falls by a large factor."""
    rng = np.random.default_rng(2)
    blocks = _blocks("rotated_column", 40, rng)
    per_token = _rel_mse(blocks, 4, 0)
    balanced = _rel_mse(blocks, 4, 2)
    assert balanced < per_token / 4


def test_variants_against_wider_codes():
    """What page balancing buys over the decode workloads' key and value
    distributions, against spending bytes on wider codes: the balanced keys
    cost 8 bytes per token and KV head (one scale byte per channel per
    16-token page), 4-bit values 16."""
    rng = np.random.default_rng(3)
    rows = []
    for kind in ("normal", "outlier_channels", "student_t3", "channel_offsets"):
        blocks = _blocks(kind, 60, rng)
        k0, k2 = _rel_mse(blocks, 4, 0), _rel_mse(blocks, 4, 2)
        v0, v2, v4 = _rel_mse(blocks, 2, 0), _rel_mse(blocks, 2, 2), _rel_mse(blocks, 4, 0)
        rows.append((kind, k0, k2, v0, v2, v4))
        if kind == "channel_offsets":
            assert k2 < 0.9 * k0 and v2 < 0.8 * v0
        else:       # columns the rotation evened out: within 1% of per-token
            assert abs(k2 / k0 - 1) < 0.01 and abs(v2 / v0 - 1) < 0.01
        assert v4 < v2 / 5
    print("\nrelative MSE          K4 per-token  K4 balanced  V2 per-token  V2 balanced  V4 per-token")
    for kind, k0, k2, v0, v2, v4 in rows:
        print(f"{kind:20s} {k0:12.3e} {k2:12.3e} {v0:13.3e} {v2:12.3e} {v4:13.3e}")
