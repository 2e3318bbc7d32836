"""Pins of the CPU oracle against facts fixed outside it.

Nothing here re-types the oracle's formulas: each check is a closed form, an
invariant, a special case that reduces to a library routine (numpy's binary16
conversion, torch's scaled-dot-product attention), brute force, or a
hand-derived fixture under tests/golden/.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import kvq_inputs as inp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128
SCALE = 1.0 / math.sqrt(128)


def _read_fixture(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = [s.strip() for s in line.split("=", 1)]
            out[k] = v
    return out


def sylvester(n=128):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


H = sylvester()


# --------------------------------------------------------------------------
# binary16 conversions vs numpy
# --------------------------------------------------------------------------

def test_half_to_double_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.signbit(got[~np.isnan(ref)]), np.signbit(ref[~np.isnan(ref)]))


def test_float_to_half_matches_numpy_rne():
    rng = np.random.default_rng(7)
    vals = [
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-5).astype(np.float32),      # subnormal range
        (rng.standard_normal(2000) * 3e4).astype(np.float32),       # near overflow
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24,
                  2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 6.1e-5, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, np.inf, -np.inf], dtype=np.float32),
    ]
    # exact ties between neighbouring binary16 values
    hb = np.arange(0x0001, 0x7bff, 97, dtype=np.uint16)
    lo = hb.view(np.float16).astype(np.float64)
    hi = (hb + 1).view(np.float16).astype(np.float64)
    vals.append(((lo + hi) / 2).astype(np.float32))
    x = np.concatenate(vals)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


# --------------------------------------------------------------------------
# Hadamard rotation
# --------------------------------------------------------------------------

def test_hadamard_entries_closed_form():
    Ho = np.array([[oracle.hadamard_entry(i, j) for j in range(D)] for i in range(D)])
    assert np.array_equal(Ho, H)                       # Sylvester recursion
    assert np.array_equal(Ho @ Ho.T, 128 * np.eye(D, dtype=np.int64))
    assert np.array_equal(Ho, Ho.T)


def test_fwht_columns_and_involution():
    for j in range(D):
        e = np.zeros(D, np.float32)
        e[j] = 1.0
        assert np.array_equal(oracle.fwht_f32(e), H[:, j].astype(np.float32))
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 9, D).astype(np.float32)
    assert np.array_equal(oracle.fwht_f32(oracle.fwht_f32(x)), 128 * x)


def test_fwht_f32_close_to_exact_on_fp16_inputs():
    rng = np.random.default_rng(2)
    for _ in range(50):
        x16 = (rng.standard_normal(D) * rng.choice([1e-3, 1, 30])).astype(np.float16)
        exact = H @ (x16.astype(np.float64))          # exact: fp16 values sum in < 53 bits
        got = oracle.fwht_f32(x16.astype(np.float32)).astype(np.float64)
        bound = 7 * 2.0 ** -24 * np.abs(x16.astype(np.float64)).sum()
        assert np.max(np.abs(got - exact)) <= bound


def test_matvec_f64():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(D)
    assert np.allclose(oracle.hadamard_matvec_f64(x), H @ x, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Encoder
# --------------------------------------------------------------------------

def _dequant(codes, s, z, bits=4):
    """Rotated-domain dequantisation: s*c + zero, where the stored offset is
    the zero itself for 4-bit keys and the group mean for 2-bit values."""
    zero = oracle.group_zero(codes, s, z, is_value=(bits == 2))
    return oracle.half_to_double(s) * codes.astype(np.float64) + zero


def test_zero_and_constant_groups():
    codes, s, z = oracle.quantize_group(np.zeros(D, np.float16), 4)
    assert not codes.any() and s == 0 and z == 0
    e0 = np.zeros(D, np.float16)
    e0[0] = 1
    for bits in (4, 2):
        codes, s, z = oracle.quantize_group(e0, bits)   # H e0 = all ones -> M == m
        assert not codes.any() and s == 0 and z == 0x3C00


def test_hand_derived_example():
    f = _read_fixture("quantize_e0_e1.txt")
    x = np.zeros(D, np.float16)
    x[0] = x[1] = 1
    for bits, pre in ((4, "key"), (2, "value")):
        codes, s, z = oracle.quantize_group(x, bits)
        assert np.all(codes[0::2] == int(f[pre + "_codes_even"]))
        assert np.all(codes[1::2] == int(f[pre + "_codes_odd"]))
        off = "_z" if pre == "key" else "_mean"
        assert s == int(f[pre + "_s"], 16) and z == int(f[pre + off], 16)


def _on_grid(rng, L, delta=2.0 ** -4, zero=-0.5):
    """fp16 group whose rotation lies exactly on an L-level grid.  Groups whose
    exact mean zero + delta * sum(c) / 128 is 0 are redrawn: the value mean is
    evaluated in fp32 from rounded normalised operands, and fp16 keeps the
    ~2^-24 residual of that cancellation as a subnormal (see
    test_value_mean_cancellation_stays_tiny), so such a group is not stored
    exactly."""
    c = rng.integers(0, L + 1, D)
    c[rng.integers(D)] = 0
    c[rng.integers(D)] = L
    while c.min() != 0 or c.max() != L or zero + delta * c.sum() / 128 == 0:
        c = rng.integers(0, L + 1, D)
    y = zero + delta * c                               # rotated-domain values, on the grid
    x = (H @ y) / 128.0                                # H^-1 = H / 128
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x)  # representable exactly
    return x16, c, delta, zero


@pytest.mark.parametrize("bits", [4, 2])
def test_on_grid_round_trip_exact(bits):
    rng = np.random.default_rng(10 + bits)
    L = (1 << bits) - 1
    for _ in range(40):
        x16, c, delta, zero = _on_grid(rng, L)
        codes, s, z = oracle.quantize_group(x16, bits)
        assert np.array_equal(codes, c)
        assert oracle.half_to_double(s) == delta
        if bits == 4:
            assert oracle.half_to_double(z) == zero
        else:   # values store the group mean, zero + delta * sum(c) / 128
            assert oracle.half_to_double(z) == zero + delta * c.sum() / 128
        assert np.array_equal(_dequant(codes, s, z, bits), zero + delta * c)


@pytest.mark.parametrize("bits", [4, 2])
def test_error_bound_and_brute_force_nearest_level(bits):
    rng = np.random.default_rng(20 + bits)
    L = (1 << bits) - 1
    levels = np.arange(L + 1, dtype=np.float64)
    for trial in range(300):
        scale = [1.0, 0.01, 50.0][trial % 3]
        x = rng.standard_normal(D) * scale
        if trial % 5 == 0:
            x[rng.integers(0, D, 3)] *= 20                   # outlier channels
        x16 = x.astype(np.float16)
        y = H @ x16.astype(np.float64)                       # exact rotation
        codes, s16, z16 = oracle.quantize_group(x16, bits)
        s = oracle.half_to_double(s16)
        z = oracle.group_zero(codes, s16, z16, is_value=(bits == 2))
        assert codes.max() <= L
        rec = s * codes + z
        slack = 2.0 ** -10 * (L * s + abs(z)) + 1e-6 * np.abs(y).max()
        err = np.abs(y - rec)
        assert np.all(err <= s / 2 + slack)
        # brute force: the chosen level is (up to the rounding slack) the nearest
        best = np.min(np.abs(y[:, None] - (s * levels[None, :] + z)), axis=1)
        assert np.all(err <= best + slack)
        assert codes[np.argmin(y)] == 0 and codes[np.argmax(y)] == L


@pytest.mark.parametrize("bits", [4, 2])
def test_scale_equivariance(bits):
    """min/max RTN is equivariant to a power-of-two input scale: codes are
    unchanged and (s, z) scale exactly (powers of two commute with every
    rounding away from over/underflow)."""
    rng = np.random.default_rng(30 + bits)
    for _ in range(100):
        # magnitudes in [0.01, 4]: every scaled copy stays a normal fp16
        x16 = (rng.choice([-1, 1], D) * rng.uniform(0.01, 4, D)).astype(np.float16)
        c0, s0, z0 = oracle.quantize_group(x16, bits)
        for k in (-3, -1, 1, 4):
            xk = (x16.astype(np.float64) * 2.0 ** k).astype(np.float16)
            assert np.array_equal(xk.astype(np.float64), x16.astype(np.float64) * 2.0 ** k)
            ck, sk, zk = oracle.quantize_group(xk, bits)
            assert np.array_equal(ck, c0)
            assert oracle.half_to_double(sk) == oracle.half_to_double(s0) * 2.0 ** k
            assert oracle.half_to_double(zk) == oracle.half_to_double(z0) * 2.0 ** k


def test_rotation_spreads_key_outliers():
    """Tiny workload keys (4 channels x20): quantising in the rotated domain
    gives a lower reconstruction error than plain min/max RTN of the raw
    channels at the same bit width."""
    w = inp.workload("tiny")
    k, _ = inp.sequence_kv(w, 0, 0, 256)
    k = k[:, 0, :].numpy()
    err_rot, err_raw = 0.0, 0.0
    for t in range(k.shape[0]):
        x = k[t].astype(np.float64)
        codes, s, z = oracle.quantize_group(k[t], 4)
        xr = (H @ _dequant(codes, s, z, 4)) / 128.0
        err_rot += np.sum((xr - x) ** 2)
        lo, hi = x.min(), x.max()
        step = (hi - lo) / 15
        xq = lo + step * np.clip(np.rint((x - lo) / step), 0, 15)
        err_raw += np.sum((xq - x) ** 2)
    assert err_rot < 0.5 * err_raw


def test_value_mean_is_dequantised_channel_zero():
    """The stored value offset is the group mean in the rotated domain, which
    equals channel 0 of the dequantised, un-rotated vector (H 1 = 128 e_0),
    and it lies within the fp16 rounding of the exact mean of y / 128."""
    rng = np.random.default_rng(50)
    region = np.zeros(1664, np.uint8)
    for trial in range(100):
        x16 = (rng.standard_normal(D) * [0.01, 1, 40][trial % 3]).astype(np.float16)
        kc, ks, kz = oracle.quantize_group(x16, 4)
        vc, vs, vmu = oracle.quantize_group(x16, 2)
        oracle.store_token(region, 3, kc, ks, kz, vc, vs, vmu)
        _, v = oracle.dequant_slot(region, 3)
        assert abs(v[0] - oracle.half_to_double(vmu)) <= 1e-12 * max(1.0, abs(v[0]))
        # the mean of the rotated values is x_0; quantisation moves it by at most s/2
        s = oracle.half_to_double(vs)
        assert abs(oracle.half_to_double(vmu) - float(x16[0])) <= s / 2 + 2.0 ** -10 * (3 * s + abs(float(x16[0]))) + 1e-7


def _on_grid_loose_zero(rng, L, delta=2.0):
    """fp16 group whose rotation y = z0 + delta * c lies exactly on an L-level
    grid, but whose zero z0 is NOT representable in fp16, while the group mean
    x_0 = z0 + delta * sum(c) / 128 (= original channel 0, since H 1 = 128 e_0)
    is.  With delta = 2 every other channel x_j = delta (H c)_j / 128 is a
    multiple of 2^-6 below 2^5 (fp16-exact), and the zero, between 16 and 32
    in magnitude for typical codes, has more bits than fp16 keeps there."""
    while True:
        c = rng.integers(0, L + 1, D)
        c[rng.integers(D)] = 0
        c[rng.integers(D)] = L
        if c.min() != 0 or c.max() != L:
            continue
        x0 = int(rng.integers(-1000, 1000)) * 2.0 ** -10
        z0 = x0 - delta * c.sum() / 128.0
        z16 = float(np.float16(z0))
        if z16 == z0:
            continue
        # stay clear of fp16 rounding midpoints: the encoder's fp32 value of z0
        # carries a rounding error of a few 2^-24 relative
        ulp = 2.0 ** (math.floor(math.log2(abs(z0))) - 10)
        if abs(abs(z16 - z0) - ulp / 2) < ulp / 64:
            continue
        y = z0 + delta * c
        x = (H @ y) / 128.0
        x16 = x.astype(np.float16)
        if not np.array_equal(x16.astype(np.float64), x):
            continue
        return x16, c, delta, z0, x0


def test_value_mean_reconstructs_channel_zero_exactly_where_the_zero_cannot():
    """The reason values store the group mean mu instead of the zero z (the
    fold of the zero-points into output channel 0 at read-back: dothoosh.com,
    "KVarN vs TurboQuant", pipeline list, stage 4).  On-grid groups whose
    rotated zero z0 is not fp16-representable: the same codes and scale come
    out in both offset modes, but
      - with mu stored, the dequantised rotated group is y exactly
        (dequant_slot_rotated) and the un-rotated one is x exactly, channel 0
        included (dequant_slot);
      - with z stored, every channel j >= 1 is still exact (H 1 = 128 e_0 keeps
        the zero out of them) but channel 0 is off by |fp16(z0) - z0| > 0.
    k4v4 holds both modes at the same width: 4-bit keys store z, 4-bit values
    mu.  The 2-bit values of K4V2 are checked the same way."""
    rng = np.random.default_rng(4242)
    err_z = []
    for trial in range(60):
        x16, c, delta, z0, x0 = _on_grid_loose_zero(rng, 15)
        kc, ks, kz = oracle.quantize_group(x16, 4, offset_mode=0)
        vc, vs, vmu = oracle.quantize_group(x16, 4, offset_mode=1)
        assert np.array_equal(kc, c) and np.array_equal(vc, c)
        assert oracle.half_to_double(ks) == delta == oracle.half_to_double(vs)
        assert oracle.half_to_double(kz) == float(np.float16(z0)) != z0
        assert oracle.half_to_double(vmu) == x0
        region = np.zeros(oracle.region_bytes((4, 4)), np.uint8)
        oracle.store_token(region, trial % 16, kc, ks, kz, vc, vs, vmu, fmt=(4, 4))
        kr, vr = oracle.dequant_slot_rotated(region, trial % 16, fmt=(4, 4))
        y = z0 + delta * c
        assert np.array_equal(vr, y)
        assert np.array_equal(kr, float(np.float16(z0)) + delta * c)
        k, v = oracle.dequant_slot(region, trial % 16, fmt=(4, 4))
        x = x16.astype(np.float64)
        assert np.array_equal(v, x)
        assert np.array_equal(k[1:], x[1:])
        assert k[0] != x[0] and abs(k[0] - x[0]) == abs(float(np.float16(z0)) - z0)
        err_z.append(abs(k[0] - x[0]))
    assert min(err_z) > 0 and max(err_z) <= 2.0 ** -7     # half an fp16 ulp at |z0| < 32
    # the K4V2 value layout (2-bit codes, mean stored): exact as well
    for trial in range(30):
        x16, c, delta, z0, x0 = _on_grid_loose_zero(rng, 3)
        vc, vs, vmu = oracle.quantize_group(x16, 2)
        assert np.array_equal(vc, c) and oracle.half_to_double(vs) == delta
        assert oracle.half_to_double(vmu) == x0
        region = np.zeros(1664, np.uint8)
        zc = np.zeros(D, np.uint8)
        oracle.store_token(region, 5, zc, 0, 0, vc, vs, vmu)
        _, vr = oracle.dequant_slot_rotated(region, 5)
        _, v = oracle.dequant_slot(region, 5)
        assert np.array_equal(vr, z0 + delta * c)
        assert np.array_equal(v, x16.astype(np.float64))


# --------------------------------------------------------------------------
# Byte layout
# --------------------------------------------------------------------------

def test_layout_golden():
    f = _read_fixture("layout_pattern.txt")
    off = int(f["off"])
    region = np.zeros(1664, np.uint8)
    kc = np.arange(D) % 16
    vc = np.arange(D) % 4
    oracle.store_token(region, off, kc, 0x1234, 0x5678, vc, 0x9ABC, 0xDEF0)
    expect = np.zeros(1664, np.uint8)
    expect[320:384] = np.frombuffer(bytes.fromhex(f["key_bytes_at_320"]), np.uint8)
    for w, o in zip(f["value_words"].split(), f["value_word_offsets"].split()):
        v = int(w, 16)
        expect[int(o)] = v & 0xFF
        expect[int(o) + 1] = v >> 8
    expect[1556:1560] = np.frombuffer(bytes.fromhex(f["key_meta_at_1556"]), np.uint8)
    expect[1620:1624] = np.frombuffer(bytes.fromhex(f["value_meta_at_1620"]), np.uint8)
    assert np.array_equal(region, expect)


def test_layout_round_trip_and_isolation():
    rng = np.random.default_rng(40)
    region = np.full(1664, 0xA5, np.uint8)
    tokens = {}
    for off in rng.permutation(16):
        kc = rng.integers(0, 16, D)
        vc = rng.integers(0, 4, D)
        meta = [int(v) for v in rng.integers(0, 65536, 4)]
        before = region.copy()
        oracle.store_token(region, int(off), kc, meta[0], meta[1], vc, meta[2], meta[3])
        changed = np.nonzero(before != region)[0]
        # a token owns 64 + 32 + 4 + 4 bytes; nothing outside them changes
        own = set(range(64 * off, 64 * off + 64))
        g, i = off // 4, off % 4
        for m in range(16):
            own |= {1024 + 128 * g + 8 * m + 2 * i, 1024 + 128 * g + 8 * m + 2 * i + 1}
        own |= set(range(1536 + 4 * off, 1540 + 4 * off)) | set(range(1600 + 4 * off, 1604 + 4 * off))
        assert set(changed.tolist()) <= own
        tokens[int(off)] = (kc, meta, vc)
    for off, (kc, meta, vc) in tokens.items():
        kc2, ks, kz, vc2, vs, vz = oracle.load_token(region, off)
        assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)
        assert [ks, kz, vs, vz] == meta


# --------------------------------------------------------------------------
# Append
# --------------------------------------------------------------------------

def test_append_is_per_token_and_idempotent():
    w = inp.workload("tiny", context=64)
    k, v = inp.sequence_kv(w, 0)
    k, v = k.numpy(), v.numpy()
    bt, npages = inp.page_table(w)
    slots = inp.slot_mapping(bt, 0, 0, 64)
    pool_a = np.full((npages, 1, 1664), 0x5A, np.uint8)
    oracle.quantize_append(k, v, slots, pool_a)
    # one token at a time, in reverse order, into a differently-filled pool
    pool_b = np.full_like(pool_a, 0x00)
    for t in reversed(range(64)):
        oracle.quantize_append(k[t:t + 1], v[t:t + 1], slots[t:t + 1], pool_b)
    assert np.array_equal(pool_a, pool_b)
    # re-append is idempotent; skipped slots (-1) write nothing
    snap = pool_a.copy()
    oracle.quantize_append(k, v, slots, pool_a)
    assert np.array_equal(pool_a, snap)
    oracle.quantize_append(k, v, np.full(64, -1, np.int64), pool_a)
    assert np.array_equal(pool_a, snap)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _small_case(num_seqs=2, hq=4, hkv=2, lens=(37, 70), seed=5, on_grid=False, page_perm=None):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int64)
    pages = [int(np.ceil(n / 16)) for n in lens]
    total = sum(pages)
    perm = rng.permutation(total) if page_perm is None else page_perm
    bt = np.full((num_seqs, max(pages)), -1, np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    pool = np.zeros((total, hkv, 1664), np.uint8)
    ks, vs = [], []
    for b in range(num_seqs):
        n = int(lens[b])
        if on_grid:
            k = np.stack([[_on_grid(rng, 15)[0] for _ in range(hkv)] for _ in range(n)])
            v = np.stack([[_on_grid(rng, 3)[0] for _ in range(hkv)] for _ in range(n)])
        else:
            k = rng.standard_normal((n, hkv, D)).astype(np.float16)
            v = rng.standard_normal((n, hkv, D)).astype(np.float16)
        oracle.quantize_append(k, v, inp.slot_mapping(bt, b, 0, n), pool)
        ks.append(k)
        vs.append(v)
    q = rng.standard_normal((num_seqs, hq, D)).astype(np.float16)
    return pool, bt, lens, q, ks, vs


def test_attention_on_grid_equals_sdpa_on_originals():
    """On-grid keys/values survive quantisation exactly, so attention over the
    quantised cache must equal textbook attention (torch SDPA, fp64) over the
    original fp16 tensors -- pins dequantisation, un-rotation, page walk and
    the GQA head mapping."""
    pool, bt, lens, q, ks, vs = _small_case(on_grid=True, seed=6)
    scale = 1 / np.sqrt(D)
    out = oracle.decode_attention(pool, bt, lens, q, scale)
    G = q.shape[1] // pool.shape[1]
    for b in range(len(lens)):
        K = torch.from_numpy(ks[b].astype(np.float64)).permute(1, 0, 2)   # [Hkv][n][D]
        V = torch.from_numpy(vs[b].astype(np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(G, 0).contiguous()
        V = V.repeat_interleave(G, 0).contiguous()
        Q = torch.from_numpy(q[b].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, 0, :]
        assert np.max(np.abs(out[b] - ref.numpy())) < 1e-12


def test_attention_folded_equals_plain():
    pool, bt, lens, q, _, _ = _small_case(seed=7, lens=(1, 129))
    scale = 1 / np.sqrt(D)
    a = oracle.decode_attention(pool, bt, lens, q, scale)
    b = oracle.decode_attention_folded(pool, bt, lens, q, scale)
    assert np.max(np.abs(a - b)) < 1e-9


def test_attention_special_cases():
    pool, bt, lens, q, _, _ = _small_case(seed=8, lens=(1, 50))
    scale = 1 / np.sqrt(D)
    out = oracle.decode_attention(pool, bt, lens, q, scale)
    # n = 1: the output is the single cached value, dequantised and un-rotated
    _, v0 = oracle.dequant_slot(pool[bt[0, 0], 0], 0)
    _, v0b = oracle.dequant_slot(pool[bt[0, 0], 1], 0)
    assert np.allclose(out[0, 0], v0, atol=1e-12) and np.allclose(out[0, 1], v0, atol=1e-12)
    assert np.allclose(out[0, 2], v0b, atol=1e-12)
    # q = 0: uniform weights -> mean of the cached values
    q0 = np.zeros_like(q)
    out0 = oracle.decode_attention(pool, bt, lens, q0, scale)
    vals = np.stack([oracle.dequant_slot(pool[bt[1, t // 16], 0], t % 16)[1] for t in range(50)])
    assert np.allclose(out0[1, 0], vals.mean(0), atol=1e-12)
    # output is a convex combination of the cached values
    assert np.all(out[1, 0] <= vals.max(0) + 1e-12) and np.all(out[1, 0] >= vals.min(0) - 1e-12)
    # a very large scale makes the softmax hard: output -> value of the best key
    keys = np.stack([oracle.dequant_slot(pool[bt[1, t // 16], 0], t % 16)[0] for t in range(50)])
    logits = keys @ q[1, 0].astype(np.float64)
    best = np.argsort(logits)[-2:]
    if logits[best[1]] - logits[best[0]] > 1e-3:
        hard = oracle.decode_attention(pool, bt, lens, q, 1e5)
        assert np.allclose(hard[1, 0], vals[best[1]], atol=1e-9)


def test_attention_identical_tokens_give_that_value():
    rng = np.random.default_rng(9)
    n = 40
    k1 = rng.standard_normal((1, 1, D)).astype(np.float16)
    v1 = rng.standard_normal((1, 1, D)).astype(np.float16)
    k = np.repeat(k1, n, 0)
    v = np.repeat(v1, n, 0)
    bt = np.array([[2, 0, 1]], np.int32)
    pool = np.zeros((3, 1, 1664), np.uint8)
    oracle.quantize_append(k, v, inp.slot_mapping(bt, 0, 0, n), pool)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    out = oracle.decode_attention(pool, bt, np.array([n]), q, 0.1)
    _, vd = oracle.dequant_slot(pool[2, 0], 0)
    assert np.allclose(out[0, 0], vd, atol=1e-12)


def test_attention_invariant_to_physical_page_placement():
    a = _small_case(seed=11, page_perm=np.arange(8))
    b = _small_case(seed=11, page_perm=np.array([5, 3, 7, 0, 6, 1, 4, 2]))
    scale = 1 / np.sqrt(D)
    oa = oracle.decode_attention(a[0], a[1], a[2], a[3], scale)
    ob = oracle.decode_attention(b[0], b[1], b[2], b[3], scale)
    assert np.array_equal(oa, ob)


# --------------------------------------------------------------------------
# Uncompressed fp16 reference attention
# --------------------------------------------------------------------------

def test_attention_f16_matches_torch_sdpa_fp64():
    """The plain fp64 attention over fp16 tokens equals torch's scaled
    dot-product attention run in fp64 on the same values (an independent
    implementation), for several lengths and GQA group sizes."""
    rng = np.random.default_rng(7)
    for n, G, qs in ((1, 1, 1.0), (17, 4, 2.0), (300, 8, 0.5), (1000, 2, 3.0)):
        k = (rng.standard_normal((n, D)) * rng.choice([0.5, 2.0])).astype(np.float16)
        v = rng.standard_normal((n, D)).astype(np.float16)
        q = (rng.standard_normal((G, D)) * qs).astype(np.float16)
        scale = 1 / math.sqrt(D)
        got = oracle.attention_f16(k, v, q, scale)
        kt = torch.from_numpy(k.astype(np.float64))[None, None].expand(1, G, n, D)
        vt = torch.from_numpy(v.astype(np.float64))[None, None].expand(1, G, n, D)
        qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0].numpy()
        assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_f16_special_cases():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((50, D)).astype(np.float16)
    v = rng.standard_normal((50, D)).astype(np.float16)
    # one token: the output is that token's value
    out = oracle.attention_f16(k[:1], v[:1], rng.standard_normal((3, D)).astype(np.float16), 0.1)
    assert np.array_equal(out, np.repeat(v[:1].astype(np.float64), 3, 0))
    # q = 0: uniform weights, the mean of the values
    out = oracle.attention_f16(k, v, np.zeros((1, D), np.float16), 0.1)
    assert np.max(np.abs(out[0] - v.astype(np.float64).mean(0))) < 1e-14
    # no tokens: zero rows
    out = oracle.attention_f16(k[:0], v[:0], np.ones((2, D), np.float16), 0.1)
    assert np.array_equal(out, np.zeros((2, D)))


def test_attention_f64_matches_torch_sdpa_and_concatenation():
    """fp64 attention over arbitrary rows equals torch SDPA (fp64), and
    attention over a union of two token sets equals the softmax-weighted merge
    of the two sets' own attentions (the log-sum-exp identity the split and
    mixed-cache decode rely on)."""
    rng = np.random.default_rng(9)
    n1, n2, G = 40, 70, 3
    k = rng.standard_normal((n1 + n2, D)) * 0.7
    v = rng.standard_normal((n1 + n2, D))
    q = rng.standard_normal((G, D)).astype(np.float16)
    scale = 1 / math.sqrt(D)
    got = oracle.attention_f64(k, v, q, scale)
    kt = torch.from_numpy(k)[None, None].expand(1, G, n1 + n2, D)
    vt = torch.from_numpy(v)[None, None].expand(1, G, n1 + n2, D)
    qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0].numpy()
    assert np.max(np.abs(got - ref)) < 1e-12
    # merge of the two halves by their log-sum-exp weights
    qd = q.astype(np.float64)
    parts = []
    for lo, hi in ((0, n1), (n1, n1 + n2)):
        lg = scale * qd @ k[lo:hi].T                     # [G][n]
        parts.append((np.log(np.exp(lg).sum(1)), oracle.attention_f64(k[lo:hi], v[lo:hi], q, scale)))
    w = np.exp(np.stack([p[0] for p in parts]))          # [2][G]
    merged = (w[0][:, None] * parts[0][1] + w[1][:, None] * parts[1][1]) / (w[0] + w[1])[:, None]
    assert np.max(np.abs(merged - got)) < 1e-12



# --------------------------------------------------------------------------
# Other bit widths: 8-bit or 4-bit keys, 4-bit or 2-bit values
# --------------------------------------------------------------------------

PRESETS = [(4, 2), (4, 4), (8, 2), (8, 4), (3, 3)]


def test_region_sizes():
    # key codes 16 x 16*kbits, value codes 16 x 16*vbits, 2 x 16 x 4 metadata
    for kb, vb in PRESETS:
        assert oracle.region_bytes((kb, vb)) == 16 * (16 * kb + 16 * vb + 8)
    assert oracle.region_bytes((4, 2)) == 1664
    with pytest.raises(ValueError):
        oracle.region_bytes((3, 2))


def test_layout_golden_k8v4():
    f = _read_fixture("layout_k8v4.txt")
    off, size = int(f["off"]), int(f["region_bytes"])
    region = np.zeros(size, np.uint8)
    c = np.arange(D)
    kc = 2 * c + 1
    vc = (c // 16 + c % 16) % 16
    oracle.store_token(region, off, kc, 0x1234, 0x5678, vc, 0x9ABC, 0xDEF0, fmt=(8, 4))
    expect = np.zeros(size, np.uint8)
    ko = int(f["key_row_offset"])
    expect[ko:ko + D] = np.arange(1, 256, 2)
    base = int(f["value_word_base"])
    for h in (0, 1):
        for m, w in enumerate(f[f"value_words_h{h}"].split()):
            v = int(w, 16)
            expect[base + 16 * m + 4 * h] = v & 0xFF
            expect[base + 16 * m + 4 * h + 1] = v >> 8
    expect[3096:3100] = np.frombuffer(bytes.fromhex(f["key_meta_at_3096"]), np.uint8)
    expect[3160:3164] = np.frombuffer(bytes.fromhex(f["value_meta_at_3160"]), np.uint8)
    assert np.array_equal(region, expect)


def test_layout_golden_k3v3():
    """3-bit codes as bit planes, against the hand-derived image of one slot."""
    f = _read_fixture("layout_k3v3.txt")
    off, size = int(f["off"]), int(f["region_bytes"])
    region = np.zeros(size, np.uint8)
    c = np.arange(D)
    kc = (c % 8) ^ (c // 32)
    vc = (c // 16) ^ (c % 16 % 8)
    oracle.store_token(region, off, kc, 0x1234, 0x5678, vc, 0x9ABC, 0xDEF0, fmt=(3, 3))
    expect = np.zeros(size, np.uint8)
    ko = int(f["key_row_offset"])
    for G in range(4):
        planes = [int(b, 16) for b in f[f"key_plane_bytes_G{G}"].split()]
        for p in range(3):
            expect[ko + 12 * G + 4 * p:ko + 12 * G + 4 * p + 4] = planes[p]
    vb = int(f["value_byte_base"])
    for m in range(16):
        planes = [int(b, 16) for b in f[f"value_plane_bytes_m{m % 8}"].split()]
        for p in range(3):
            expect[vb + 12 * m + 4 * p] = planes[p]
    expect[1556:1560] = np.frombuffer(bytes.fromhex(f["key_meta_at_1556"]), np.uint8)
    expect[1620:1624] = np.frombuffer(bytes.fromhex(f["value_meta_at_1620"]), np.uint8)
    assert np.array_equal(region, expect)


def test_layout_k4_keys_are_the_k4v2_keys():
    """Key rows do not depend on the value width: 4-bit keys in the 4/4 layout
    are byte-identical to the 4/2 layout's (pinned by layout_pattern.txt)."""
    rng = np.random.default_rng(41)
    kc = rng.integers(0, 16, D)
    a = np.zeros(1664, np.uint8)
    b = np.zeros(oracle.region_bytes((4, 4)), np.uint8)
    oracle.store_token(a, 9, kc, 1, 2, np.zeros(D, np.uint8), 3, 4)
    oracle.store_token(b, 9, kc, 1, 2, np.zeros(D, np.uint8), 3, 4, fmt=(4, 4))
    assert np.array_equal(a[:1024], b[:1024])


@pytest.mark.parametrize("fmt", PRESETS)
def test_layout_round_trip_and_isolation_presets(fmt):
    kb, vb = fmt
    size = oracle.region_bytes(fmt)
    rng = np.random.default_rng(42 + kb + vb)
    region = np.full(size, 0xA5, np.uint8)
    tokens = {}
    owned = np.zeros(size, np.int64)
    for off in rng.permutation(16):
        kc = rng.integers(0, 1 << kb, D)
        vc = rng.integers(0, 1 << vb, D)
        meta = [int(v) for v in rng.integers(0, 65536, 4)]
        before = region.copy()
        oracle.store_token(region, int(off), kc, meta[0], meta[1], vc, meta[2], meta[3], fmt=fmt)
        # a token owns exactly 16*(kbits + vbits) + 8 bytes, disjoint from every other token's
        tokens[int(off)] = (kc, meta, vc)
        assert np.count_nonzero(before != region) <= 16 * (kb + vb) + 8
    for off, (kc, meta, vc) in tokens.items():
        kc2, ks, kz, vc2, vs, vz = oracle.load_token(region, off, fmt=fmt)
        assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)
        assert [ks, kz, vs, vz] == meta
    # ownership: flipping one token's codes changes only its own bytes
    for off in range(16):
        kc, meta, vc = tokens[off]
        before = region.copy()
        oracle.store_token(region, off, (1 << kb) - 1 - kc, meta[0] ^ 0xFFFF, meta[1] ^ 0xFFFF,
                           (1 << vb) - 1 - vc, meta[2] ^ 0xFFFF, meta[3] ^ 0xFFFF, fmt=fmt)
        diff = np.nonzero(before != region)[0]
        assert diff.size == 16 * (kb + vb) + 8          # every owned bit flipped
        owned[diff] += 1
        for o2, (kc2, meta2, vc2) in tokens.items():
            if o2 != off:
                assert np.array_equal(oracle.load_token(region, o2, fmt=fmt)[0], kc2)
        oracle.store_token(region, off, kc, *meta[:2], vc, *meta[2:], fmt=fmt)
    assert np.all(owned == 1)                         # the 16 tokens tile the region


def _sparse_on_grid_8bit(rng, delta=2.0 ** -4, zero=-0.5):
    """Rotated-domain group y = zero + delta * c with codes c spanning 0..255
    whose inverse rotation x = H y / 128 is sparse and fp16-exact: c_j =
    sum_r 2^r (1 - H[j, k_r]) / 2 over 8 distinct columns k_r, each of which
    has H[j*, k_r] = -1 at one row j* (so c_0 = 0 and c_j* = 255)."""
    jstar = int(rng.integers(1, D))
    cols = [k for k in range(1, D) if H[jstar, k] == -1]
    ks = rng.choice(cols, 8, replace=False)
    c = np.zeros(D, np.int64)
    for r, k in enumerate(ks):
        c += (1 << r) * (1 - H[:, k]) // 2
    assert c.min() == 0 and c.max() == 255 and c[0] == 0 and c[jstar] == 255
    y = zero + delta * c
    x = (H @ y) / 128.0
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x)
    return x16, c, delta, zero


@pytest.mark.parametrize("bits,mode", [(8, 0), (4, 1), (8, 1), (3, 0), (3, 1)])
def test_on_grid_round_trip_exact_other_widths(bits, mode):
    """8-bit keys and 4-bit (or 8-bit) groups with the value offset (the group
    mean): codes, scale and offset come back exactly."""
    rng = np.random.default_rng(60 + bits + mode)
    L = (1 << bits) - 1
    for _ in range(40):
        x16, c, delta, zero = _sparse_on_grid_8bit(rng) if bits == 8 else _on_grid(rng, L)
        codes, s, z = oracle.quantize_group(x16, bits, offset_mode=mode)
        assert np.array_equal(codes, c)
        assert oracle.half_to_double(s) == delta
        expect_off = zero if mode == 0 else zero + delta * c.sum() / 128
        assert oracle.half_to_double(z) == expect_off
        rec = oracle.half_to_double(s) * codes + oracle.group_zero(codes, s, z, is_value=(mode == 1))
        assert np.array_equal(rec, zero + delta * c)


@pytest.mark.parametrize("bits", [8, 4, 3])
def test_error_bound_and_brute_force_nearest_level_other_widths(bits):
    rng = np.random.default_rng(70 + bits)
    L = (1 << bits) - 1
    levels = np.arange(L + 1, dtype=np.float64)
    for trial in range(200):
        mode = trial % 2
        x = rng.standard_normal(D) * [1.0, 0.01, 50.0][trial % 3]
        if trial % 5 == 0:
            x[rng.integers(0, D, 3)] *= 20
        x16 = x.astype(np.float16)
        y = H @ x16.astype(np.float64)
        codes, s16, z16 = oracle.quantize_group(x16, bits, offset_mode=mode)
        s = oracle.half_to_double(s16)
        z = oracle.group_zero(codes, s16, z16, is_value=(mode == 1))
        assert codes.max() <= L
        rec = s * codes + z
        # the fp16 offset of a value group is the mean, so its rounding is
        # spread over L*s/2 at most; keys round z itself
        slack = 2.0 ** -10 * (L * s + abs(z)) + 1e-6 * np.abs(y).max()
        err = np.abs(y - rec)
        assert np.all(err <= s / 2 + slack)
        best = np.min(np.abs(y[:, None] - (s * levels[None, :] + z)), axis=1)
        assert np.all(err <= best + slack)
        assert codes[np.argmin(y)] == 0 and codes[np.argmax(y)] == L


def test_wider_codes_lower_the_error():
    """Same groups at 2, 3, 4 and 8 bits: the mean squared reconstruction
    error falls by about 4x per extra bit (uniform quantiser, step ~ range /
    L, so the ratio between widths is about (L_wide / L_narrow)^2)."""
    rng = np.random.default_rng(80)
    err = {2: 0.0, 3: 0.0, 4: 0.0, 8: 0.0}
    for _ in range(200):
        x16 = rng.standard_normal(D).astype(np.float16)
        y = H @ x16.astype(np.float64)
        for bits in err:
            codes, s, z = oracle.quantize_group(x16, bits, offset_mode=1)
            rec = oracle.half_to_double(s) * codes + oracle.group_zero(codes, s, z, is_value=True)
            err[bits] += np.mean((y - rec) ** 2)
    assert err[4] < err[2] / 16 * 2.5 and err[4] > err[2] / 16 / 2.5
    assert err[3] < err[2] / (7 / 3) ** 2 * 2.5 and err[3] > err[2] / (7 / 3) ** 2 / 2.5
    assert err[4] < err[3] / (15 / 7) ** 2 * 2.5 and err[4] > err[3] / (15 / 7) ** 2 / 2.5
    assert err[8] < err[4] / 256 * 2.5


@pytest.mark.parametrize("fmt", [(4, 4), (8, 2), (8, 4), (3, 3)])
def test_append_per_token_and_idempotent_presets(fmt):
    w = inp.workload("tiny", context=48)
    k, v = inp.sequence_kv(w, 0)
    k, v = k.numpy(), v.numpy()
    bt, npages = inp.page_table(w)
    slots = inp.slot_mapping(bt, 0, 0, 48)
    size = oracle.region_bytes(fmt)
    pool_a = np.full((npages, 1, size), 0x5A, np.uint8)
    oracle.quantize_append(k, v, slots, pool_a, fmt=fmt)
    pool_b = np.zeros_like(pool_a)
    for t in reversed(range(48)):
        oracle.quantize_append(k[t:t + 1], v[t:t + 1], slots[t:t + 1], pool_b, fmt=fmt)
    assert np.array_equal(pool_a, pool_b)
    # the codes and metadata stored are the group encoder's at the preset's widths
    for t in (0, 17, 47):
        page, off = slots[t] // 16, slots[t] % 16
        kc, ks, kz, vc, vs, vz = oracle.load_token(pool_a[page, 0], off, fmt=fmt)
        assert (kc.tolist(), ks, kz) == _tolist(oracle.quantize_group(k[t, 0], fmt[0], offset_mode=0))
        assert (vc.tolist(), vs, vz) == _tolist(oracle.quantize_group(v[t, 0], fmt[1], offset_mode=1))


def _tolist(g):
    return g[0].tolist(), g[1], g[2]


def _small_case_fmt(fmt, num_seqs=2, hq=4, hkv=2, lens=(37, 70), seed=5, on_grid=False):
    rng = np.random.default_rng(seed)
    kb, vb = fmt
    pages = [int(np.ceil(n / 16)) for n in lens]
    perm = rng.permutation(sum(pages))
    bt = np.full((num_seqs, max(pages)), -1, np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    pool = np.zeros((sum(pages), hkv, oracle.region_bytes(fmt)), np.uint8)
    ks, vs = [], []
    for b in range(num_seqs):
        n = int(lens[b])
        if on_grid:
            gk = (lambda: _sparse_on_grid_8bit(rng)[0]) if kb == 8 else (lambda: _on_grid(rng, (1 << kb) - 1)[0])
            k = np.stack([[gk() for _ in range(hkv)] for _ in range(n)])
            v = np.stack([[_on_grid(rng, (1 << vb) - 1)[0] for _ in range(hkv)] for _ in range(n)])
        else:
            k = rng.standard_normal((n, hkv, D)).astype(np.float16)
            v = rng.standard_normal((n, hkv, D)).astype(np.float16)
        oracle.quantize_append(k, v, inp.slot_mapping(bt, b, 0, n), pool, fmt=fmt)
        ks.append(k)
        vs.append(v)
    q = rng.standard_normal((num_seqs, hq, D)).astype(np.float16)
    return pool, bt, np.asarray(lens, np.int64), q, ks, vs


@pytest.mark.parametrize("fmt", [(4, 4), (8, 2), (8, 4), (3, 3)])
def test_attention_on_grid_equals_sdpa_presets(fmt):
    pool, bt, lens, q, ks, vs = _small_case_fmt(fmt, on_grid=True, seed=9)
    scale = 1 / np.sqrt(D)
    out = oracle.decode_attention(pool, bt, lens, q, scale, fmt=fmt)
    G = q.shape[1] // pool.shape[1]
    for b in range(len(lens)):
        K = torch.from_numpy(ks[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        V = torch.from_numpy(vs[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        Q = torch.from_numpy(q[b].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[:, 0, :]
        assert np.max(np.abs(out[b] - ref.numpy())) < 1e-12


@pytest.mark.parametrize("fmt", [(4, 4), (8, 2), (8, 4), (3, 3)])
def test_attention_folded_equals_plain_presets(fmt):
    pool, bt, lens, q, _, _ = _small_case_fmt(fmt, seed=11, lens=(1, 129))
    scale = 1 / np.sqrt(D)
    a = oracle.decode_attention(pool, bt, lens, q, scale, fmt=fmt)
    b = oracle.decode_attention_folded(pool, bt, lens, q, scale, fmt=fmt)
    assert np.max(np.abs(a - b)) < 1e-9


# --------------------------------------------------------------------------
# Several query rows per sequence (causal)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [(4, 2), (8, 4)])
def test_attention_mq_on_grid_equals_causal_sdpa(fmt):
    """On-grid K/V survive quantisation exactly, so the multi-row decode must
    equal torch SDPA (fp64) with a causal mask aligned to the sequence end,
    over the original tensors."""
    M = 5
    pool, bt, lens, _, ks, vs = _small_case_fmt(fmt, on_grid=True, seed=21, lens=(37, 70))
    rng = np.random.default_rng(22)
    B, Hkv = len(lens), pool.shape[1]
    Hq = 4
    G = Hq // Hkv
    q = rng.standard_normal((B, M, Hq, D)).astype(np.float16)
    scale = 1 / np.sqrt(D)
    out = oracle.decode_attention_mq(pool, bt, lens, q, scale, fmt=fmt)
    for b in range(B):
        n = int(lens[b])
        K = torch.from_numpy(ks[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        V = torch.from_numpy(vs[b].astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
        Q = torch.from_numpy(q[b].astype(np.float64)).permute(1, 0, 2).contiguous()      # [Hq][M][D]
        mask = torch.arange(n)[None, :] <= (n - M + torch.arange(M))[:, None]            # [M][n]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
        assert np.max(np.abs(out[b] - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_attention_mq_rows_are_truncated_single_decodes():
    pool, bt, lens, _, _, _ = _small_case(num_seqs=3, seed=23, lens=(20, 33, 1))
    rng = np.random.default_rng(24)
    M, Hq = 3, 4
    q = rng.standard_normal((3, M, Hq, D)).astype(np.float16)
    scale = 1 / np.sqrt(D)
    out = oracle.decode_attention_mq(pool, bt, lens, q, scale)
    for m in range(M):
        trunc = np.maximum(lens - M + m + 1, 0)
        ref = oracle.decode_attention(pool, bt, trunc, q[:, m], scale)
        for b in range(3):
            if trunc[b] == 0:
                assert not out[b, m].any()            # a row that sees no token is zero
            else:
                assert np.max(np.abs(out[b, m] - ref[b])) < 1e-13
    one = oracle.decode_attention_mq(pool, bt, lens, q[:, :1], scale)
    assert np.max(np.abs(one[:, 0] - oracle.decode_attention(pool, bt, lens, q[:, 0], scale))) < 1e-13


def test_value_mean_cancellation_stays_tiny():
    """An on-grid value group whose exact mean is 0: the fp32 mean comes out
    within a few units of 2^-24 (the cancellation residual, kept by fp16 as a
    subnormal), far inside the quantiser's error bound s/2."""
    rng = np.random.default_rng(90)
    hits = 0
    while hits < 20:
        c = rng.integers(0, 16, D)
        c[0], c[1] = 0, 15
        c[2] += 1024 - c.sum()
        if not (0 <= c[2] <= 15):
            continue
        y = -0.5 + 2.0 ** -4 * c
        x16 = ((H @ y) / 128.0).astype(np.float16)
        if not np.array_equal(x16.astype(np.float64), (H @ y) / 128.0):
            continue
        codes, s, mu = oracle.quantize_group(x16, 4, offset_mode=1)
        assert np.array_equal(codes, c) and oracle.half_to_double(s) == 2.0 ** -4
        assert abs(oracle.half_to_double(mu)) <= 4 * 2.0 ** -24
        hits += 1


# --------------------------------------------------------------------------
# Pages of 32, 64 and 128 tokens
# --------------------------------------------------------------------------

@pytest.mark.parametrize("P,fmt", [(32, (4, 2)), (64, (8, 4)), (128, (4, 4))])
def test_larger_pages_are_relabelled_16_token_pages(P, fmt):
    """A pool of P-token pages, u8 [N][H][P/16][region], is a pool of 16-token
    pages laid out [N*P/16][H][region] with 16-token page p*S + s holding
    sub-region s of page p (S = P/16).  The append and both attention calls at
    page size P must agree with the 16-token ones under that relabelling."""
    S = P // 16
    rng = np.random.default_rng(P + fmt[0])
    B, Hq, Hkv, lens = 3, 8, 2, [P * 2 + 5, 17, P - 1]
    R = oracle.region_bytes(fmt)
    pages = [-(-n // P) for n in lens]
    N = sum(pages) + 1
    perm = rng.permutation(N)
    bt = np.zeros((B, max(pages)), np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    # the 16-token relabelling of the same pages
    bt16 = np.zeros((B, max(pages) * S), np.int32)
    for b in range(B):
        for j in range(pages[b] * S):
            bt16[b, j] = bt[b, j // S] * S + j % S
    pool = np.zeros((N, Hkv, S * R), np.uint8)
    pool16 = np.zeros((N * S, Hkv, R), np.uint8)
    for b, n in enumerate(lens):
        k = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        t = np.arange(n)
        oracle.quantize_append(k, v, bt[b, t // P].astype(np.int64) * P + t % P, pool, fmt=fmt, page_tokens=P)
        oracle.quantize_append(k, v, bt16[b, t // 16].astype(np.int64) * 16 + t % 16, pool16, fmt=fmt)
    relabelled = pool.reshape(N, Hkv, S, R).transpose(0, 2, 1, 3).reshape(N * S, Hkv, R)
    assert np.array_equal(relabelled, pool16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    a = oracle.decode_attention(pool, bt, np.array(lens), q, SCALE, fmt=fmt, page_tokens=P)
    b16 = oracle.decode_attention(pool16, bt16, np.array(lens), q, SCALE, fmt=fmt)
    assert np.array_equal(a, b16)
    qm = rng.standard_normal((B, 3, Hq, D)).astype(np.float16)
    am = oracle.decode_attention_mq(pool, bt, np.array(lens), qm, SCALE, fmt=fmt, page_tokens=P)
    bm = oracle.decode_attention_mq(pool16, bt16, np.array(lens), qm, SCALE, fmt=fmt)
    assert np.array_equal(am, bm)
