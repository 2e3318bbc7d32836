"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: packed cache bytes bit-identical to the oracle's; attention max-abs error
<= 2e-3 against the oracle's fp64 plain-definition attention (fp32 or fp16
output).  Small cases are checked in full; the five workloads at full size in
the launch configuration the benchmark uses, on sampled (sequence, KV head)
groups that the oracle recomputes from the same seeded inputs.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import kvq_inputs as inp
import oracle
import quantized_decode_attention_quantize_amd as kvq

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

TOL = 2e-3
D = 128
SCALE = 1.0 / math.sqrt(D)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.load()
    return torch.device("cuda:0")


def log(msg):
    print(msg, flush=True)


def valid_byte_mask(n_tokens_in_page: int) -> np.ndarray:
    """Bytes of a region that hold data of the first r token slots."""
    r = n_tokens_in_page
    m = np.zeros(1664, bool)
    m[:64 * r] = True
    for o in range(r):
        for mm in range(16):
            off = 1024 + 128 * (o // 4) + 8 * mm + 2 * (o % 4)
            m[off:off + 2] = True
    m[1536:1536 + 4 * r] = True
    m[1600:1600 + 4 * r] = True
    return m


def gpu_append(k, v, slots, cache, fmt=None):
    kvq.quantize_append(k, v, slots, cache, fmt=fmt)


# bit widths (keys, values) of the quantised presets; (4, 2) is KVarN's
PRESET_FMTS = [(4, 4), (8, 2), (8, 4), (3, 3)]


def _kfmt(fmt):
    """The library's format of (kbits, vbits), None for the default (4, 2)."""
    return None if tuple(fmt) == (4, 2) else kvq.format_from_string(f"k{fmt[0]}v{fmt[1]}_g128")


# --------------------------------------------------------------------------
# Quantise-append
# --------------------------------------------------------------------------

def test_append_tiny_workload_bit_exact(dev):
    w = inp.workload("tiny")
    n = int(inp.final_lens(w)[0])
    bt, num_pages = inp.page_table(w)
    k, v = inp.sequence_kv(w, 0)
    slots = inp.slot_mapping(bt, 0, 0, n)
    log(f"append tiny n={n} pages={num_pages}")
    cache = torch.full((num_pages, 1, 1664), 0xA5, dtype=torch.uint8, device=dev)
    gpu_append(k.to(dev), v.to(dev), torch.from_numpy(slots).to(dev), cache)
    pool = np.full((num_pages, 1, 1664), 0xA5, np.uint8)
    oracle.quantize_append(k.numpy(), v.numpy(), slots, pool)
    assert np.array_equal(cache.cpu().numpy(), pool)


def _mixed_tokens(rng, T, H):
    """fp16 [T][H][128] rows drawn from several regimes, including subnormal
    inputs, large values, outlier channels, zero rows, rows whose rotation is
    constant, and near-tie rows built on a half-step grid."""
    Hm = np.array([[1]])
    while Hm.shape[0] < D:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    x = np.empty((T, H, D), np.float64)
    kinds = rng.integers(0, 8, (T, H))
    for t in range(T):
        for h in range(H):
            kd = kinds[t, h]
            if kd == 0:
                r = rng.standard_normal(D)
            elif kd == 1:
                r = rng.standard_normal(D) * 1e-5               # fp16 subnormals
            elif kd == 2:
                r = rng.standard_normal(D) * 300.0
            elif kd == 3:
                r = rng.standard_normal(D)
                r[rng.integers(0, D, 4)] *= 20.0
            elif kd == 4:
                r = np.zeros(D)
            elif kd == 5:
                r = np.zeros(D)
                r[0] = rng.choice([-3.0, 0.5, 7.25])          # rotation is constant
            elif kd == 6:                                     # half-step grid: ties
                L = 15 if rng.random() < 0.5 else 3
                hs = rng.integers(0, 2 * L + 1, D)
                hs[0], hs[1] = 0, 2 * L
                y = -0.5 + hs * (2.0 ** -5)
                r = (Hm @ y) / 128.0
            else:
                r = rng.standard_t(3, D)
            x[t, h] = r
    return x.astype(np.float16)


# The last case has 65600 (token, KV head) rows, which selects the bulk
# one-lane-per-group kernel; the others run the 16-lane kernel.
@pytest.mark.parametrize("H,T,num_pages,seed", [(1, 37, 8, 1), (3, 200, 20, 2), (8, 515, 40, 3),
                                                (8, 8200, 600, 4)])
def test_append_mixed_regimes_strided_and_skips(dev, H, T, num_pages, seed):
    rng = np.random.default_rng(100 + seed)
    log(f"append mixed H={H} T={T} pages={num_pages}")
    k = _mixed_tokens(rng, T, H)
    v = _mixed_tokens(rng, T, H)
    slots = rng.permutation(num_pages * 16)[:T].astype(np.int64)
    slots[rng.integers(0, T, 5)] = -1                          # skipped tokens
    slots[0] = num_pages * 16 + 3                               # outside the pool: skipped
    # strided inputs: token stride (H + 1) * 128
    kb = torch.zeros((T, H + 1, D), dtype=torch.float16)
    vb = torch.zeros((T, H + 1, D), dtype=torch.float16)
    kb[:, :H] = torch.from_numpy(k)
    vb[:, :H] = torch.from_numpy(v)
    kd, vd = kb.to(dev)[:, :H], vb.to(dev)[:, :H]
    cache = torch.full((num_pages, H, 1664), 0x3C, dtype=torch.uint8, device=dev)
    gpu_append(kd, vd, torch.from_numpy(slots).to(dev), cache)
    pool = np.full((num_pages, H, 1664), 0x3C, np.uint8)
    ok = (slots >= 0) & (slots < num_pages * 16)
    oracle.quantize_append(k[ok], v[ok], slots[ok], pool)
    got = cache.cpu().numpy()
    diff = np.argwhere(got != pool)
    assert diff.size == 0, f"{len(diff)} bytes differ, first at {diff[:5].tolist()}"


# Bulk appends (65536 (token, KV head) rows and more) take the LDS-staged
# kernel for power-of-two head counts -- with separate address forms below 4
# heads, from 4 to 32, and 64 or more -- and the lane-per-row kernel
# otherwise.  (H, T, token-stride padding in elements, format)
BULK = [(1, 65600, 0, (4, 2)), (2, 33000, 8, (4, 2)), (4, 17000, 0, (4, 2)), (8, 8193, 24, (4, 2)),
        (16, 4200, 0, (8, 4)), (64, 1100, 0, (4, 2)), (128, 520, 16, (4, 4)), (3, 22000, 0, (4, 2)),
        (8, 8300, 0, (3, 3)), (8, 8300, 8, (8, 2))]


@pytest.mark.parametrize("H,T,pad,fmt", BULK)
def test_bulk_append_kernels_bit_exact(dev, H, T, pad, fmt):
    """Bulk appends against the oracle, bit for bit, over the whole pool:
    random page placement, strided token rows, skipped slots (negative) and
    slots outside the pool (not written), and a ragged last batch."""
    log(f"bulk append H={H} T={T} pad={pad} fmt={fmt}")
    rng = np.random.default_rng(H * 1000 + T + pad)
    region, kf = oracle.region_bytes(fmt), _kfmt(fmt)
    num_pages = -(-T // 16) + 3
    perm = rng.permutation(num_pages).astype(np.int64)
    t = np.arange(T)
    slots = perm[t // 16] * 16 + t % 16
    slots[rng.choice(T, 37, replace=False)] = -1
    slots[rng.choice(T, 11, replace=False)] = (num_pages + 2) * 16 + 3       # outside the pool
    width = H * D + pad
    kbuf = (rng.standard_normal((T, width)) * rng.choice([0.05, 1, 30], (T, 1))).astype(np.float16)
    vbuf = rng.standard_normal((T, width)).astype(np.float16)
    kbuf[:, 5::97] *= 12
    kt, vt = torch.from_numpy(kbuf).to(dev), torch.from_numpy(vbuf).to(dev)
    k = kt[:, :H * D].view(T, H, D) if pad == 0 else torch.as_strided(kt, (T, H, D), (width, D, 1))
    v = vt[:, :H * D].view(T, H, D) if pad == 0 else torch.as_strided(vt, (T, H, D), (width, D, 1))
    cache = torch.full((num_pages, H, region), 0xA5, dtype=torch.uint8, device=dev)
    gpu_append(k, v, torch.from_numpy(slots).to(dev), cache, fmt=kf)
    pool = np.full((num_pages, H, region), 0xA5, np.uint8)
    in_pool = np.where(slots < num_pages * 16, slots, -1)        # the oracle skips them the same way
    oracle.quantize_append(np.ascontiguousarray(kbuf[:, :H * D].reshape(T, H, D)),
                           np.ascontiguousarray(vbuf[:, :H * D].reshape(T, H, D)), in_pool, pool, fmt=fmt)
    got = cache.cpu().numpy()
    if not np.array_equal(got, pool):
        bad = np.argwhere(got != pool)
        raise AssertionError(f"{len(bad)} bytes differ, first at (page, head, byte) {bad[0].tolist()}")


def test_append_one_token_at_a_time_matches_bulk(dev):
    w = inp.workload("qwen3_32b_16k", context=64, new_tokens=0, num_seqs=2)
    bt, num_pages = inp.page_table(w)
    caches = []
    for mode in ("bulk", "single"):
        cache = torch.zeros((num_pages, w.num_kv_heads, 1664), dtype=torch.uint8, device=dev)
        for b in range(w.num_seqs):
            k, v = inp.sequence_kv(w, b, device=dev)
            slots = torch.from_numpy(inp.slot_mapping(bt, b, 0, 64)).to(dev)
            if mode == "bulk":
                gpu_append(k, v, slots, cache)
            else:
                for t in range(64):
                    gpu_append(k[t:t + 1], v[t:t + 1], slots[t:t + 1], cache)
        caches.append(cache.cpu())
    assert torch.equal(caches[0], caches[1])


# --------------------------------------------------------------------------
# Decode attention, small cases in full
# --------------------------------------------------------------------------

def _build_case(dev, B, Hq, Hkv, lens, seed, spare_pages=3, fmt=(4, 2)):
    rng = np.random.default_rng(seed)
    region = oracle.region_bytes(fmt)
    lens = np.asarray(lens, np.int64)
    pages = [int(math.ceil(n / 16)) for n in lens]
    num_pages = sum(pages) + spare_pages
    perm = rng.permutation(num_pages)
    max_pages = max(pages) + 2
    bt = np.full((B, max_pages), -1, np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    cache = torch.full((num_pages, Hkv, region), 0xFF, dtype=torch.uint8, device=dev)  # NaN metadata in unused slots
    pool = np.full((num_pages, Hkv, region), 0xFF, np.uint8)
    for b in range(B):
        n = int(lens[b])
        k = (rng.standard_normal((n, Hkv, D)) * rng.choice([0.5, 1, 2])).astype(np.float16)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        k[:, :, rng.integers(0, D, 3)] *= 10
        slots = inp.slot_mapping(bt, b, 0, n)
        gpu_append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                   torch.from_numpy(slots).to(dev), cache, fmt=_kfmt(fmt))
        oracle.quantize_append(k, v, slots, pool, fmt=fmt)
    q = (rng.standard_normal((B, Hq, D)) * rng.choice([0.5, 1, 3])).astype(np.float16)
    return cache, pool, bt, lens, q


SMALL = [
    # B, Hq, Hkv, lens
    (1, 1, 1, [1]),
    (1, 1, 1, [15]),
    (1, 2, 1, [16]),
    (2, 4, 1, [17, 33]),
    (2, 8, 2, [31, 32]),
    (3, 8, 1, [100, 1, 257]),
    (2, 16, 2, [1000, 999]),
    (1, 32, 2, [700]),        # G = 16: two head groups
    (4, 12, 4, [64, 65, 127, 300]),   # G = 3
    (2, 64, 8, [513, 77]),
]


@pytest.mark.parametrize("B,Hq,Hkv,lens", SMALL)
def test_decode_small_matches_oracle(dev, B, Hq, Hkv, lens):
    log(f"decode small B={B} Hq={Hq} Hkv={Hkv} lens={lens}")
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, lens, seed=B * 1000 + Hq + sum(lens))
    assert np.array_equal(cache.cpu().numpy(), pool)
    ref = oracle.decode_attention(pool, bt, lens_np, q, SCALE)
    qd = torch.from_numpy(q).to(dev)
    btd = torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    for pps in (0, 2, 6):
        out = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=pps)
        err = np.max(np.abs(out.cpu().numpy() - ref))
        assert err <= TOL, f"pps={pps} err={err}"
    out16 = kvq.decode_attention(qd, cache, btd, ld, L, out_dtype=torch.float16)
    err16 = np.max(np.abs(out16.float().cpu().numpy() - ref))
    assert err16 <= TOL, f"fp16 out err={err16}"


# Sequence lengths whose waves run 4 to 16 page pairs per split at 128 pages per
# split (64 pairs over 4 waves): whole unguarded rounds of three pairs, every
# length (1 to 4 pairs) of the guarded last stretch, the work-left priority steps
# and a masked last pair.  With 16 query heads per KV head (two head groups) the
# guarded loop runs throughout.
LOOP_LENS = [600, 700, 800, 900, 1000, 1100, 1300, 2049, 4000]


@pytest.mark.parametrize("Hq,Hkv,fmt", [(8, 1, (4, 2)), (32, 2, (4, 2)), (16, 2, (4, 4))])
def test_decode_pair_loop_lengths_match_oracle(dev, Hq, Hkv, fmt):
    B = len(LOOP_LENS)
    log(f"decode pair-loop lengths Hq={Hq} Hkv={Hkv} fmt={fmt} lens={LOOP_LENS}")
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, LOOP_LENS, seed=4099 + Hq + fmt[1], fmt=fmt)
    assert np.array_equal(cache.cpu().numpy(), pool)
    ref = oracle.decode_attention(pool, bt, lens_np, q, SCALE, fmt=fmt)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    for pps in (128, 64, 0):
        out = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=pps, fmt=_kfmt(fmt))
        err = np.max(np.abs(out.cpu().numpy() - ref))
        assert err <= TOL, f"pps={pps} err={err}"


def test_decode_deterministic_split_invariant_and_page_placement(dev):
    B, Hq, Hkv, lens = 3, 16, 2, [400, 1, 777]
    log("decode determinism / split / placement")
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, lens, seed=77)
    qd = torch.from_numpy(q).to(dev)
    btd = torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    ws = kvq.alloc_workspace(B, Hq, Hkv, L)
    a = kvq.decode_attention(qd, cache, btd, ld, L, workspace=ws).cpu()
    b = kvq.decode_attention(qd, cache, btd, ld, L, workspace=ws).cpu()
    assert torch.equal(a, b)                         # repeat: identical bits, workspace reused
    c = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=2).cpu()
    assert torch.max(torch.abs(a - c)).item() <= 1e-5
    # move every page to another physical slot; same logical cache
    num_pages = cache.shape[0]
    rng = np.random.default_rng(5)
    newpos = rng.permutation(num_pages)
    cache2 = torch.empty_like(cache)
    cache2[torch.from_numpy(newpos).to(dev)] = cache
    bt2 = np.where(bt >= 0, newpos[np.maximum(bt, 0)], -1).astype(np.int32)
    d = kvq.decode_attention(qd, cache2, torch.from_numpy(bt2).to(dev), ld, L, workspace=ws).cpu()
    assert torch.equal(a, d)


@pytest.mark.parametrize("lens,pps", [([400, 1, 777], 0), ([400, 1, 777], 2), ([20, 0, 50], 0),
                                      ([20, 0, 50], 4)])
def test_decode_two_phase_matches_fused(dev, lens, pps):
    """kvq_decode_partials + kvq_decode_combine give the bits of
    kvq_decode_attention_ex, also for single-split and empty sequences."""
    B, Hq, Hkv = len(lens), 16, 2
    log(f"decode two-phase lens={lens} pps={pps}")
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, [max(n, 1) for n in lens], seed=31)
    lens_np = np.asarray(lens, np.int64)
    qd = torch.from_numpy(q).to(dev)
    btd = torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    for dt in (torch.float32, torch.float16):
        fused = kvq.decode_attention(qd, cache, btd, ld, L, out_dtype=dt, pages_per_split=pps).cpu()
        ws = kvq.alloc_workspace(B, Hq, Hkv, L, pps)
        ws.fill_(0xA5)                                # any contents
        kvq.decode_partials(qd, cache, btd, ld, L, ws, pages_per_split=pps)
        two = kvq.decode_combine(ws, ld, Hq, Hkv, L, out_dtype=dt, pages_per_split=pps).cpu()
        assert torch.equal(fused, two), f"dtype={dt}"
        for b, n in enumerate(lens):
            if n == 0:
                assert torch.count_nonzero(two[b]).item() == 0
    ref = oracle.decode_attention(pool, bt, np.maximum(lens_np, 1), q, SCALE)
    for b, n in enumerate(lens):
        if n:
            assert np.max(np.abs(two[b].float().numpy() - ref[b])) <= TOL


FUSED = [
    # B, Hq, Hkv, lens including the new token, pages_per_split
    (1, 8, 1, [1], 0),
    (2, 8, 1, [16, 17], 0),
    (3, 16, 2, [400, 33, 777], 0),
    (3, 16, 2, [400, 32, 776], 2),      # new token fills a page inside the pair loop
    (2, 32, 2, [300, 129], 0),          # G = 16: both head groups in one work-group
    (2, 64, 8, [513, 64], 4),
    # G = 32: four head groups, two work-groups per (split, KV head), each of
    # which encodes the new token into the same slot before reading the page
    (2, 64, 2, [300, 129], 0),
    (3, 64, 2, [40, 17, 1], 2),
]


@pytest.mark.parametrize("B,Hq,Hkv,lens,pps,fmt", [c + ((4, 2),) for c in FUSED] +
                         [FUSED[2] + (f,) for f in PRESET_FMTS] + [FUSED[5] + (f,) for f in PRESET_FMTS])
def test_fused_append_decode_matches_two_calls(dev, B, Hq, Hkv, lens, pps, fmt):
    """kvq_append_decode_attention (and its partials + combine form) leaves the
    cache bytes and the output of kvq_quantize_append followed by
    kvq_decode_attention_ex, bit for bit, and both match the oracle."""
    log(f"fused append+decode B={B} Hq={Hq} Hkv={Hkv} lens={lens} pps={pps} fmt={fmt}")
    rng = np.random.default_rng(B * 7919 + Hq + sum(lens) + pps)
    region, kf = oracle.region_bytes(fmt), _kfmt(fmt)
    pages = [int(math.ceil(n / 16)) for n in lens]
    num_pages = sum(pages) + 2
    perm = rng.permutation(num_pages)
    bt = np.full((B, max(pages) + 1), -1, np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    cache = torch.full((num_pages, Hkv, region), 0xFF, dtype=torch.uint8, device=dev)
    pool = np.full((num_pages, Hkv, region), 0xFF, np.uint8)
    new_k = np.zeros((B, Hkv, D), np.float16)
    new_v = np.zeros((B, Hkv, D), np.float16)
    for b, n in enumerate(lens):
        k = (rng.standard_normal((n, Hkv, D)) * rng.choice([0.5, 2])).astype(np.float16)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        k[:, :, rng.integers(0, D, 3)] *= 10
        new_k[b], new_v[b] = k[n - 1], v[n - 1]
        if n > 1:
            slots = inp.slot_mapping(bt, b, 0, n - 1)
            gpu_append(torch.from_numpy(k[:n - 1]).to(dev), torch.from_numpy(v[:n - 1]).to(dev),
                       torch.from_numpy(slots).to(dev), cache, fmt=kf)
            oracle.quantize_append(k[:n - 1], v[:n - 1], slots, pool, fmt=fmt)
    q = (rng.standard_normal((B, Hq, D)) * 2).astype(np.float16)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.tensor(lens, dtype=torch.int32, device=dev)
    nkd, nvd = torch.from_numpy(new_k).to(dev), torch.from_numpy(new_v).to(dev)
    L = max(lens)
    last_slots = np.array([bt[b, (n - 1) // 16] * 16 + (n - 1) % 16 for b, n in enumerate(lens)], np.int64)
    cache_b, cache_c = cache.clone(), cache.clone()
    # two calls
    gpu_append(nkd, nvd, torch.from_numpy(last_slots).to(dev), cache, fmt=kf)
    out_a = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=pps, fmt=kf).cpu()
    # fused, one call
    out_b = kvq.append_decode_attention(nkd, nvd, qd, cache_b, btd, ld, L, pages_per_split=pps, fmt=kf).cpu()
    assert torch.equal(cache.cpu(), cache_b.cpu()), "fused append changed other bytes or encoded differently"
    assert torch.equal(out_a, out_b)
    # fused split phase + combine, fp16 output
    ws = kvq.alloc_workspace(B, Hq, Hkv, L, pps, fmt=kf)
    kvq.append_decode_partials(nkd, nvd, qd, cache_c, btd, ld, L, ws, pages_per_split=pps, fmt=kf)
    out_c = kvq.decode_combine(ws, ld, Hq, Hkv, L, out_dtype=torch.float16, pages_per_split=pps, fmt=kf).cpu()
    out_a16 = kvq.decode_attention(qd, cache, btd, ld, L, out_dtype=torch.float16, pages_per_split=pps,
                                   fmt=kf).cpu()
    assert torch.equal(cache.cpu(), cache_c.cpu())
    assert torch.equal(out_a16, out_c)
    # the oracle
    oracle.quantize_append(new_k, new_v, last_slots, pool, fmt=fmt)
    assert np.array_equal(cache.cpu().numpy(), pool)
    ref = oracle.decode_attention(pool, bt, np.asarray(lens), q, SCALE, fmt=fmt)
    assert np.max(np.abs(out_b.numpy() - ref)) <= TOL


def test_fused_append_page_outside_pool_is_skipped(dev):
    """A new token whose page id lies outside the pool is not stored by either
    path; both read page 0 in its place and agree bit for bit."""
    B, Hq, Hkv, lens = 2, 8, 1, [40, 20]
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, lens, seed=4242)
    bt = bt.copy()
    bt[1, 1] = cache.shape[0] + 3                     # sequence 1's last page: outside the pool
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    rng = np.random.default_rng(3)
    nk = torch.from_numpy(rng.standard_normal((B, Hkv, D)).astype(np.float16)).to(dev)
    nv = torch.from_numpy(rng.standard_normal((B, Hkv, D)).astype(np.float16)).to(dev)
    cache_b = cache.clone()
    slots = torch.tensor([bt[b, (n - 1) // 16] * 16 + (n - 1) % 16 for b, n in enumerate(lens)],
                         dtype=torch.int64, device=dev)
    gpu_append(nk, nv, slots, cache)
    out_a = kvq.decode_attention(qd, cache, btd, ld, 40).cpu()
    out_b = kvq.append_decode_attention(nk, nv, qd, cache_b, btd, ld, 40).cpu()
    assert torch.equal(cache.cpu(), cache_b.cpu())
    assert torch.equal(out_a, out_b)


def test_split_kernel_events_hook(dev):
    """kvq_set_split_kernel_events: the split kernel records the caller's
    events at its start and end; results are unchanged, and clearing the hook
    stops the recording."""
    B, Hq, Hkv, lens = 2, 16, 2, [300, 77]
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, lens, seed=99)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(e0)) == 0 and hip.hipEventCreate(ctypes.byref(e1)) == 0
    lib = kvq.load()
    plain = kvq.decode_attention(qd, cache, btd, ld, 300).cpu()
    assert lib.kvq_set_split_kernel_events(e0, e1) == 0
    try:
        timed = kvq.decode_attention(qd, cache, btd, ld, 300).cpu()
    finally:
        assert lib.kvq_set_split_kernel_events(None, None) == 0
    torch.cuda.synchronize()
    t = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(t), e0, e1) == 0
    assert 0.0 < t.value < 100.0
    assert torch.equal(plain, timed)
    hip.hipEventDestroy(e0)
    hip.hipEventDestroy(e1)


@pytest.mark.parametrize("n16", [1, 7, 4096, 1000003])
def test_stream_read_probe_reads_every_word(dev, n16):
    """kvq_stream_read_probe (the bench's measured read ceiling) reads every
    16-byte word: one marked word anywhere in the buffer reaches the sink."""
    lib = kvq.load()
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    mark = np.int32(np.uint32(0x9E3779B9).view(np.int32))
    log(f"stream read probe n16={n16}")
    for w in sorted({0, 3, (n16 // 2) * 4 + 1, n16 * 4 - 1}):
        buf.zero_()
        sink.zero_()
        buf[w] = int(mark)
        st = lib.kvq_stream_read_probe(ctypes.c_void_p(buf.data_ptr()), n16 * 16,
                                       ctypes.c_void_p(sink.data_ptr()), None)
        assert st == 0
        assert int(sink.cpu()[0]) == int(mark), f"word {w} not read"
    buf.zero_()
    sink.zero_()
    assert lib.kvq_stream_read_probe(ctypes.c_void_p(buf.data_ptr()), n16 * 16,
                                     ctypes.c_void_p(sink.data_ptr()), None) == 0
    assert int(sink.cpu()[0]) == 0


def test_page_walk_probe_reads_the_decode_regions(dev):
    """kvq_page_walk_probe (the bench's page-walk ceiling) reads every word of
    every region the decode reads, and no other: a marked word in a region of
    a block-table page reaches the sink; one in a page that no block table
    names does not.  Page counts are even, so no page is read twice (a lone
    last page is read as both halves of its pair, like the decode's)."""
    lib = kvq.load()
    fmt = kvq.format_from_string()
    B, Hkv, num_pages, maxp, pps = 2, 2, 64, 40, 8
    lens = [16 * 40, 16 * 17 + 5]                       # 40 and 18 pages
    perm = np.random.default_rng(5).permutation(num_pages - 2)   # ids 62, 63 never named
    bt = np.zeros((B, maxp), np.int32)
    bt[0, :40] = perm[:40]
    bt[1, :18] = perm[40:58]
    pool = torch.zeros((num_pages, Hkv, 1664), dtype=torch.uint8, device=dev)
    words = pool.view(torch.int32)                      # [page][head][416]
    bt_d = torch.from_numpy(bt).to(dev)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    mark = int(np.uint32(0x9E3779B9).view(np.int32))
    P = ctypes.c_void_p
    cases = [((int(bt[0, 0]), 0, 0), True), ((int(bt[0, 39]), 1, 415), True), ((int(bt[1, 17]), 1, 200), True),
             ((int(bt[1, 5]), 0, 103), True), ((62, 0, 5), False), ((63, 1, 415), False)]
    for (page, head, w), read in cases:
        log(f"page walk probe mark page={page} head={head} word={w} read={read}")
        words.zero_()
        sink.zero_()
        words[page, head, w] = mark
        st = lib.kvq_page_walk_probe(ctypes.byref(fmt), P(pool.data_ptr()), num_pages, P(bt_d.data_ptr()), maxp,
                                     P(lens_d.data_ptr()), B, Hkv, 640, pps, P(sink.data_ptr()), None)
        assert st == 0
        assert (int(sink.cpu()[0]) == mark) == read, (page, head, w)


def test_decode_zero_query_gives_mean_value(dev):
    B, Hq, Hkv, lens = 1, 4, 1, [123]
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, lens, seed=9)
    q[:] = 0
    out = kvq.decode_attention(torch.from_numpy(q).to(dev), cache, torch.from_numpy(bt).to(dev),
                               torch.from_numpy(lens_np.astype(np.int32)).to(dev), 123).cpu().numpy()
    vals = np.stack([oracle.dequant_slot(pool[bt[0, t // 16], 0], t % 16)[1] for t in range(123)])
    assert np.max(np.abs(out[0] - vals.mean(0)[None, :])) <= TOL


# --------------------------------------------------------------------------
# The workloads at full size, sampled
# --------------------------------------------------------------------------

def _fill_cache(w, dev, keep=()):
    """Append every sequence's cached tokens (positions [0, seq_lens)) on the GPU;
    returns (cache, block_tables, kept host K/V of the sequences in `keep`)."""
    bt, num_pages = inp.page_table(w)
    lens = inp.seq_lens(w)
    cache = torch.zeros((num_pages, w.num_kv_heads, 1664), dtype=torch.uint8, device=dev)
    kept = {}
    for b in range(w.num_seqs):
        n = int(lens[b])
        k, v = inp.sequence_kv(w, b, 0, n, device=dev)
        slots = torch.from_numpy(inp.slot_mapping(bt, b, 0, n)).to(dev)
        gpu_append(k, v, slots, cache)
        if b in keep:
            kept[b] = (k.cpu().numpy(), v.cpu().numpy())
        del k, v
    return cache, bt, kept


def _check_group(cache, bt, b, kvh, n, k_seq, v_seq, q_b, G, out_b):
    """Oracle check of (sequence b, KV head kvh): codes of all n tokens and the
    attention of the G query heads."""
    pages = int(math.ceil(n / 16))
    pool = np.zeros((pages, 1, 1664), np.uint8)
    oracle.quantize_append(k_seq[:n, kvh:kvh + 1], v_seq[:n, kvh:kvh + 1],
                           np.arange(n, dtype=np.int64), pool)
    ids = torch.from_numpy(bt[b, :pages].astype(np.int64)).to(cache.device)
    got = cache[ids, kvh].cpu().numpy()
    full = got[:-1] == pool[:-1, 0]
    assert full.all(), f"codes differ in full pages of seq {b} head {kvh}"
    r = n - 16 * (pages - 1)
    m = valid_byte_mask(r)
    assert np.array_equal(got[-1][m], pool[-1, 0][m]), f"codes differ in last page of seq {b} head {kvh}"
    qh = q_b[kvh * G:(kvh + 1) * G][None]
    ref = oracle.decode_attention(pool, np.arange(pages, dtype=np.int32)[None], np.array([n]), qh, SCALE)[0]
    err = np.max(np.abs(out_b[kvh * G:(kvh + 1) * G].astype(np.float64) - ref))
    assert err <= TOL, f"seq {b} kv head {kvh}: max-abs err {err}"
    return err


def _decode(w, dev, cache, bt, lens, q, out_dtype=torch.float32):
    L = int(lens.max())
    return kvq.decode_attention(q.to(dev), cache, torch.from_numpy(bt).to(dev),
                                torch.from_numpy(lens.astype(np.int32)).to(dev), L,
                                out_dtype=out_dtype)


def test_workload_tiny(dev):
    w = inp.workload("tiny")
    log("workload tiny")
    cache, bt, kept = _fill_cache(w, dev, keep=(0,))
    lens = inp.seq_lens(w)
    q = inp.queries(w)
    out = _decode(w, dev, cache, bt, lens, q).cpu().numpy()
    _check_group(cache, bt, 0, 0, int(lens[0]), *kept[0], q.numpy()[0], 1, out[0])


def test_workload_qwen3_32b_16k(dev):
    """8 x 16384 cached tokens, append one token per sequence, then decode
    16385 tokens; 64 q / 8 KV heads.  Samples 2 sequences x 2 KV heads."""
    w = inp.workload("qwen3_32b_16k")
    log("workload qwen3_32b_16k: fill")
    keep = (0, 5)
    cache, bt, kept = _fill_cache(w, dev, keep=keep)
    lens = inp.seq_lens(w)
    # the step: append token `context` of every sequence, then attend
    new_k, new_v, slots = [], [], []
    for b in range(w.num_seqs):
        k, v = inp.sequence_kv(w, b, w.context, 1)
        new_k.append(k)
        new_v.append(v)
        slots.append(inp.slot_mapping(bt, b, w.context, 1))
    kn, vn = torch.cat(new_k), torch.cat(new_v)
    gpu_append(kn.to(dev), vn.to(dev), torch.from_numpy(np.concatenate(slots)).to(dev), cache)
    lens1 = lens + 1
    q = inp.queries(w)
    log("workload qwen3_32b_16k: decode")
    out = _decode(w, dev, cache, bt, lens1, q, out_dtype=torch.float16).float().cpu().numpy()
    for b in keep:
        k, v = kept[b]
        k = np.concatenate([k, kn[b:b + 1].numpy()])
        v = np.concatenate([v, vn[b:b + 1].numpy()])
        for kvh in (0, 7):
            e = _check_group(cache, bt, b, kvh, int(lens1[b]), k, v, q.numpy()[b], w.gqa, out[b])
            log(f"  seq {b} kv {kvh}: err {e:.2e}")


def test_workload_qwen3_4b_64k_ragged(dev):
    w = inp.workload("qwen3_4b_64k")
    log("workload qwen3_4b_64k: fill")
    lens = inp.seq_lens(w)
    keep = (int(np.argmin(lens)), int(np.argmax(lens)))
    cache, bt, kept = _fill_cache(w, dev, keep=keep)
    q = inp.queries(w)
    out = _decode(w, dev, cache, bt, lens, q).cpu().numpy()
    for b in keep:
        e = _check_group(cache, bt, b, 3, int(lens[b]), *kept[b], q.numpy()[b], w.gqa, out[b])
        log(f"  seq {b} (n={lens[b]}) kv 3: err {e:.2e}")


def test_workload_qwen3_30b_a3b_128k(dev):
    w = inp.workload("qwen3_30b_a3b_128k")
    log("workload qwen3_30b_a3b_128k: fill")
    cache, bt, kept = _fill_cache(w, dev, keep=(2,))
    lens = inp.seq_lens(w)
    q = inp.queries(w)
    out = _decode(w, dev, cache, bt, lens, q).cpu().numpy()
    e = _check_group(cache, bt, 2, 1, int(lens[2]), *kept[2], q.numpy()[2], w.gqa, out[2])
    log(f"  seq 2 kv 1: err {e:.2e}")


def test_workload_llama31_70b_prefill_then_decode(dev):
    """Bulk quantise-append of a 131072-token prompt (one call), then decode
    steps that each append one token; steps 0, 1 and 63 are checked."""
    w = inp.workload("llama31_70b_128k")
    bt, num_pages = inp.page_table(w)
    n0 = w.context
    log("workload llama31_70b_128k: prefill")
    k, v = inp.sequence_kv(w, 0, 0, n0 + w.new_tokens, device=dev)
    cache = torch.zeros((num_pages, w.num_kv_heads, 1664), dtype=torch.uint8, device=dev)
    slots_all = torch.from_numpy(inp.slot_mapping(bt, 0, 0, n0 + w.new_tokens)).to(dev)
    gpu_append(k[:n0], v[:n0], slots_all[:n0], cache)
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    btd = torch.from_numpy(bt).to(dev)
    ws = kvq.alloc_workspace(1, w.num_q_heads, w.num_kv_heads, n0 + w.new_tokens)
    for step in range(w.new_tokens):
        gpu_append(k[n0 + step:n0 + step + 1], v[n0 + step:n0 + step + 1],
                   slots_all[n0 + step:n0 + step + 1], cache)
        n = n0 + step + 1
        q = inp.queries(w, step)
        lens = torch.tensor([n], dtype=torch.int32, device=dev)
        out = kvq.decode_attention(q.to(dev), cache, btd, lens, n0 + w.new_tokens, workspace=ws)
        if step in (0, 1, w.new_tokens - 1):
            e = _check_group(cache, bt, 0, 5, n, kh, vh, q.numpy()[0], w.gqa, out.cpu().numpy()[0])
            log(f"  step {step} (n={n}) kv 5: err {e:.2e}")


# --------------------------------------------------------------------------
# Uncompressed fp16 baseline cache (the reference the K4V2 format saves on)
# --------------------------------------------------------------------------

F16 = None


def _f16():
    global F16
    if F16 is None:
        F16 = kvq.format_from_string("fp16")
    return F16


def _f16_read_token(region, off):
    """Key and value rows of token slot `off` from one 8192-byte fp16 region,
    per the layout in include/kvq.h."""
    e = region.view(np.uint16)
    n = np.arange(D)
    k_idx = off * 128 + 32 * ((n >> 3) & 3) + 8 * (n >> 5) + (n & 7)
    q, i = off // 4, off % 4
    v_idx = 2048 + ((16 * q + (n & 15)) * 8 + (n >> 4)) * 4 + i
    return e[k_idx].view(np.float16), e[v_idx].view(np.float16)


def test_fp16_append_layout_round_trip(dev):
    """fp16 append stores every row bit for bit at the documented positions
    and touches nothing else (skipped and out-of-pool slots included)."""
    rng = np.random.default_rng(61)
    T, H, num_pages = 300, 3, 30
    k = rng.standard_normal((T, H, D)).astype(np.float16)
    v = rng.standard_normal((T, H, D)).astype(np.float16)
    slots = rng.permutation(num_pages * 16)[:T].astype(np.int64)
    slots[rng.integers(0, T, 4)] = -1
    slots[1] = num_pages * 16 + 7
    cache = torch.full((num_pages, H, 8192), 0xA5, dtype=torch.uint8, device=dev)
    kvq.quantize_append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), torch.from_numpy(slots).to(dev),
                        cache, fmt=_f16())
    got = cache.cpu().numpy()
    touched = np.zeros(got.shape, bool)
    for t in range(T):
        s_ = int(slots[t])
        if s_ < 0 or s_ >= num_pages * 16:
            continue
        for h in range(H):
            kk, vv = _f16_read_token(got[s_ // 16, h], s_ % 16)
            assert np.array_equal(kk.view(np.uint16), k[t, h].view(np.uint16))
            assert np.array_equal(vv.view(np.uint16), v[t, h].view(np.uint16))
    # every written byte belongs to an appended slot: count them
    written = int(np.count_nonzero(got != 0xA5))
    expected_max = int(((slots >= 0) & (slots < num_pages * 16)).sum()) * H * 512
    assert written <= expected_max


def _build_case_f16(dev, B, Hq, Hkv, lens, seed):
    rng = np.random.default_rng(seed)
    pages = [int(math.ceil(n / 16)) for n in lens]
    num_pages = sum(pages) + 2
    perm = rng.permutation(num_pages)
    bt = np.full((B, max(pages) + 1), -1, np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    # unwritten slots hold NaN bit patterns: a partial page must not read them
    cache = torch.full((num_pages, Hkv, 8192), 0xFF, dtype=torch.uint8, device=dev)
    kv = []
    for b, n in enumerate(lens):
        k = (rng.standard_normal((n, Hkv, D)) * rng.choice([0.5, 2])).astype(np.float16)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        k[:, :, rng.integers(0, D, 3)] *= 10
        slots = inp.slot_mapping(bt, b, 0, n)
        kvq.quantize_append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                            torch.from_numpy(slots).to(dev), cache, fmt=_f16())
        kv.append((k, v))
    q = (rng.standard_normal((B, Hq, D)) * rng.choice([0.5, 1, 3])).astype(np.float16)
    return cache, bt, np.asarray(lens), q, kv


def _f16_ref(kv, lens, q, Hq, Hkv):
    G = Hq // Hkv
    out = np.zeros((len(lens), Hq, D))
    for b, n in enumerate(lens):
        k, v = kv[b]
        for h in range(Hkv):
            out[b, h * G:(h + 1) * G] = oracle.attention_f16(k[:, h], v[:, h], q[b, h * G:(h + 1) * G], SCALE)
    return out


@pytest.mark.parametrize("B,Hq,Hkv,lens", SMALL)
def test_fp16_decode_small_matches_oracle(dev, B, Hq, Hkv, lens):
    log(f"fp16 decode small B={B} Hq={Hq} Hkv={Hkv} lens={lens}")
    cache, bt, lens_np, q, kv = _build_case_f16(dev, B, Hq, Hkv, lens, seed=B * 31 + Hq + sum(lens))
    ref = _f16_ref(kv, lens, q, Hq, Hkv)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    for pps in (0, 2, 6):
        out = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=pps, fmt=_f16())
        err = np.max(np.abs(out.cpu().numpy() - ref))
        assert err <= TOL, f"pps={pps} err={err}"
    out16 = kvq.decode_attention(qd, cache, btd, ld, L, out_dtype=torch.float16, fmt=_f16())
    assert np.max(np.abs(out16.float().cpu().numpy() - ref)) <= TOL
    # the two-phase form gives the same bits
    ws = kvq.alloc_workspace(B, Hq, Hkv, L, 2, fmt=_f16())
    kvq.decode_partials(qd, cache, btd, ld, L, ws, pages_per_split=2, fmt=_f16())
    two = kvq.decode_combine(ws, ld, Hq, Hkv, L, pages_per_split=2, fmt=_f16())
    one = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=2, fmt=_f16())
    assert torch.equal(one, two)


def test_fp16_decode_qwen3_32b_shape_sampled(dev):
    """The Qwen3-32B decode shape (8 x 16385 tokens, 64 / 8 heads) on the fp16
    cache: every sequence decoded; the oracle recomputes sequences 0 and 5."""
    B, Hq, Hkv, n = 8, 64, 8, 16385
    log("fp16 decode qwen3_32b shape")
    rng = np.random.default_rng(2024)
    pages = -(-n // 16)
    num_pages = B * pages
    bt = rng.permutation(num_pages).astype(np.int32).reshape(B, pages)
    cache = torch.empty((num_pages, Hkv, 8192), dtype=torch.uint8, device=dev)
    kv = {}
    for b in range(B):
        g = torch.Generator(device=dev)
        g.manual_seed(1000 + b)
        k = torch.randn((n, Hkv, D), generator=g, device=dev).half()
        v = torch.randn((n, Hkv, D), generator=g, device=dev).half()
        kvq.quantize_append(k, v, torch.from_numpy(inp.slot_mapping(bt, b, 0, n)).to(dev), cache, fmt=_f16())
        if b in (0, 5):
            kv[b] = (k.cpu().numpy(), v.cpu().numpy())
    q = (rng.standard_normal((B, Hq, D))).astype(np.float16)
    out = kvq.decode_attention(torch.from_numpy(q).to(dev), cache, torch.from_numpy(bt).to(dev),
                               torch.full((B,), n, dtype=torch.int32, device=dev), n, fmt=_f16()).cpu().numpy()
    G = Hq // Hkv
    for b in (0, 5):
        k, v = kv[b]
        for h in (0, 7):
            ref = oracle.attention_f16(k[:, h], v[:, h], q[b, h * G:(h + 1) * G], SCALE)
            assert np.max(np.abs(out[b, h * G:(h + 1) * G] - ref)) <= TOL


# --------------------------------------------------------------------------
# Mixed caches: fp16 sink + recent window beside the K4V2 history
# --------------------------------------------------------------------------

@pytest.mark.parametrize("sink,window,hist", [(4, 48, [300, 1000, 0]), (0, 16, [513, 77, 1]), (2, 1, [64, 31, 200])])
def test_mixed_fp16_window_with_k4v2_history(dev, sink, window, hist):
    """Attention over a sequence whose first `sink` and last `window` tokens
    sit uncompressed in an fp16 cache and whose other tokens sit in a K4V2
    cache: K4V2 partials and rotated fp16 partials merged by one combine equal
    the oracle's attention over the union (history dequantised, window raw)."""
    B, Hq, Hkv = len(hist), 16, 2
    G = Hq // Hkv
    log(f"mixed cache sink={sink} window={window} hist={hist}")
    rng = np.random.default_rng(sink * 131 + window + sum(hist))
    # K4V2 history cache
    cache_h, pool_h, bt_h, lens_h, q = _build_case(dev, B, Hq, Hkv, [max(n, 1) for n in hist], seed=sum(hist) + 5)
    lens_h = np.asarray(hist, np.int64)
    # fp16 window cache: sink + recent tokens of every sequence
    nf = sink + window
    pages_f = -(-max(nf, 1) // 16)
    bt_f = (np.arange(B * pages_f, dtype=np.int32).reshape(B, pages_f))
    cache_f = torch.full((B * pages_f, Hkv, 8192), 0xFF, dtype=torch.uint8, device=dev)
    kf = (rng.standard_normal((B, nf, Hkv, D)) * 0.8).astype(np.float16)
    vf = rng.standard_normal((B, nf, Hkv, D)).astype(np.float16)
    for b in range(B):
        if nf:
            kvq.quantize_append(torch.from_numpy(kf[b]).to(dev), torch.from_numpy(vf[b]).to(dev),
                                torch.from_numpy(inp.slot_mapping(bt_f, b, 0, nf)).to(dev), cache_f, fmt=_f16())
    qd = torch.from_numpy(q).to(dev)
    Lh, Lf = max(int(lens_h.max()), 1), max(nf, 1)
    s_h = kvq.decode_split_slots(B, Hq, Hkv, Lh)
    s_f = kvq.decode_split_slots(B, Hq, Hkv, Lf, fmt=_f16())
    total = s_h + s_f
    ws = torch.full((kvq.slots_workspace_bytes(B, Hq, total),), 0xFF, dtype=torch.uint8, device=dev)
    kvq.decode_partials_slots(qd, cache_h, torch.from_numpy(bt_h).to(dev),
                              torch.from_numpy(lens_h.astype(np.int32)).to(dev), Lh, ws, 0, total)
    kvq.decode_partials_slots(qd, cache_f, torch.from_numpy(bt_f).to(dev),
                              torch.full((B,), nf, dtype=torch.int32, device=dev), Lf, ws, s_h, total,
                              rotated=True, fmt=_f16())
    out = kvq.decode_combine_slots(ws, B, Hq, total).cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            kh = np.zeros((hist[b], D)); vh = np.zeros((hist[b], D))
            for t in range(hist[b]):
                kh[t], vh[t] = oracle.dequant_slot(pool_h[bt_h[b, t // 16], h], t % 16)
            k_all = np.concatenate([kf[b, :, h].astype(np.float64), kh])
            v_all = np.concatenate([vf[b, :, h].astype(np.float64), vh])
            ref = oracle.attention_f64(k_all, v_all, q[b, h * G:(h + 1) * G], SCALE)
            err = np.max(np.abs(out[b, h * G:(h + 1) * G] - ref))
            assert err <= TOL, f"b={b} h={h} err={err}"


def test_rotated_fp16_partials_alone(dev):
    """fp16 partials stored in the Hadamard domain and combined with the K4V2
    epilogue give the plain fp16 decode (to rounding)."""
    B, Hq, Hkv, lens = 2, 8, 1, [400, 33]
    cache, bt, lens_np, q, kv = _build_case_f16(dev, B, Hq, Hkv, lens, seed=77)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    plain = kvq.decode_attention(qd, cache, btd, ld, 400, fmt=_f16()).cpu().numpy()
    total = kvq.decode_split_slots(B, Hq, Hkv, 400, fmt=_f16()) + 1        # one spare slot, written below
    ws = torch.empty((kvq.slots_workspace_bytes(B, Hq, total),), dtype=torch.uint8, device=dev)
    kvq.decode_partials_slots(qd, cache, btd, ld, 400, ws, 1, total, rotated=True, fmt=_f16())
    # slot 0: an empty cache's partials (all sequences of length 0)
    kvq.decode_partials_slots(qd, cache, btd, torch.zeros(B, dtype=torch.int32, device=dev), 16, ws, 0, total,
                              rotated=True, pages_per_split=2, fmt=_f16())
    out = kvq.decode_combine_slots(ws, B, Hq, total).cpu().numpy()
    assert np.max(np.abs(out - plain)) <= 1e-5
    assert np.max(np.abs(out - _f16_ref(kv, lens, q, Hq, Hkv))) <= TOL



# --------------------------------------------------------------------------
# Other bit widths: 4/8-bit keys with 2/4-bit values, 3 bits both
# --------------------------------------------------------------------------

# 65600 (token, KV head) rows select the one-lane-per-group append kernel
@pytest.mark.parametrize("fmt", PRESET_FMTS)
@pytest.mark.parametrize("H,T,num_pages,seed", [(3, 200, 20, 12), (8, 8200, 600, 14)])
def test_preset_append_bit_exact(dev, fmt, H, T, num_pages, seed):
    rng = np.random.default_rng(300 + seed + 10 * fmt[0] + fmt[1])
    log(f"preset append fmt={fmt} H={H} T={T}")
    region = oracle.region_bytes(fmt)
    k = _mixed_tokens(rng, T, H)
    v = _mixed_tokens(rng, T, H)
    slots = rng.permutation(num_pages * 16)[:T].astype(np.int64)
    slots[rng.integers(0, T, 5)] = -1
    slots[0] = num_pages * 16 + 3
    cache = torch.full((num_pages, H, region), 0x3C, dtype=torch.uint8, device=dev)
    gpu_append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), torch.from_numpy(slots).to(dev), cache,
               fmt=_kfmt(fmt))
    pool = np.full((num_pages, H, region), 0x3C, np.uint8)
    ok = (slots >= 0) & (slots < num_pages * 16)
    oracle.quantize_append(k[ok], v[ok], slots[ok], pool, fmt=fmt)
    diff = np.argwhere(cache.cpu().numpy() != pool)
    assert diff.size == 0, f"{len(diff)} bytes differ, first at {diff[:5].tolist()}"


PRESET_SMALL = [
    (1, 1, 1, [1]),
    (2, 4, 1, [17, 33]),
    (3, 8, 1, [100, 1, 257]),
    (1, 32, 2, [700]),
    (4, 12, 4, [64, 65, 127, 300]),
    (2, 64, 8, [513, 77]),
]


@pytest.mark.parametrize("fmt", PRESET_FMTS)
@pytest.mark.parametrize("B,Hq,Hkv,lens", PRESET_SMALL)
def test_preset_decode_small_matches_oracle(dev, fmt, B, Hq, Hkv, lens):
    log(f"preset decode fmt={fmt} B={B} Hq={Hq} Hkv={Hkv} lens={lens}")
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, lens, seed=B * 1000 + Hq + sum(lens) + fmt[0],
                                              fmt=fmt)
    assert np.array_equal(cache.cpu().numpy(), pool)
    ref = oracle.decode_attention(pool, bt, lens_np, q, SCALE, fmt=fmt)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    for pps in (0, 2, 6):
        out = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=pps, fmt=_kfmt(fmt))
        err = np.max(np.abs(out.cpu().numpy() - ref))
        assert err <= TOL, f"pps={pps} err={err}"
    out16 = kvq.decode_attention(qd, cache, btd, ld, L, out_dtype=torch.float16, fmt=_kfmt(fmt))
    assert np.max(np.abs(out16.float().cpu().numpy() - ref)) <= TOL


def test_bench_step_qwen3_32b_16k_k4v2(dev):
    """The benchmark's timed step at full size: Qwen3-32B shape (8 x 16384
    cached tokens, 64 q / 8 KV heads), the cache filled by the bulk append,
    then kvq_append_decode_partials (the split kernel encodes each
    sequence's token 16384 into its page) and kvq_decode_combine, with the
    heuristic split and fp16 output, exactly as bench.py calls them.
    Checked against the oracle: the new token's bytes of every (sequence, KV
    head), all 16385 tokens' bytes of 2 sequences x 2 KV heads, and the
    attention of their 8 query heads (2e-3)."""
    w = inp.workload("qwen3_32b_16k")
    B, Hq, Hkv, ctx = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.context
    n = ctx + 1
    log("bench step qwen3_32b_16k k4v2: fill")
    bt, num_pages = inp.page_table(w)
    cache = torch.zeros((num_pages, Hkv, 1664), dtype=torch.uint8, device=dev)
    keep = (0, 5)
    kept, new_k, new_v = {}, [], []
    for b in range(B):
        k, v = inp.sequence_kv(w, b, 0, n, device=dev)
        gpu_append(k[:ctx], v[:ctx], torch.from_numpy(inp.slot_mapping(bt, b, 0, ctx)).to(dev), cache)
        new_k.append(k[ctx:])
        new_v.append(v[ctx:])
        if b in keep:
            kept[b] = (k.cpu().numpy(), v.cpu().numpy())
        del k, v
    nk, nv = torch.cat(new_k).contiguous(), torch.cat(new_v).contiguous()
    q = inp.queries(w, 0, device=dev).contiguous()
    lens = torch.full((B,), n, dtype=torch.int32, device=dev)
    btd = torch.from_numpy(bt).to(dev)
    pps = kvq.decode_pages_per_split(B, Hq, Hkv, n)
    log(f"bench step: fused partials + combine, {pps} pages per split")
    ws = kvq.alloc_workspace(B, Hq, Hkv, n)
    kvq.append_decode_partials(nk, nv, q, cache, btd, lens, n, ws)
    out = kvq.decode_combine(ws, lens, Hq, Hkv, n, out_dtype=torch.float16).float().cpu().numpy()
    torch.cuda.synchronize()
    # the appended token of every sequence and KV head
    nk_np, nv_np = nk.cpu().numpy(), nv.cpu().numpy()
    page = bt[:, ctx // 16]
    region_np = cache[torch.from_numpy(page.astype(np.int64)).to(dev)].cpu().numpy()      # [B][Hkv][1664]
    for b in range(B):
        pool = np.zeros((1, Hkv, 1664), np.uint8)
        oracle.quantize_append(nk_np[b:b + 1], nv_np[b:b + 1], np.array([ctx % 16], np.int64), pool)
        for kvh in range(Hkv):
            got, ref = region_np[b, kvh], pool[0, kvh]
            o = ctx % 16
            for lo, hi in ((64 * o, 64 * o + 64), (1536 + 4 * o, 1540 + 4 * o), (1600 + 4 * o, 1604 + 4 * o)):
                assert np.array_equal(got[lo:hi], ref[lo:hi]), f"new token of seq {b} head {kvh}"
            for g4 in range(16):      # value words of slot o: u16 at 1024 + 128 (o/4) + 8 m + 2 (o%4)
                a = 1024 + 128 * (o // 4) + 8 * g4 + 2 * (o % 4)
                assert np.array_equal(got[a:a + 2], ref[a:a + 2])
    pages = int(math.ceil(n / 16))
    for b in keep:
        k_seq, v_seq = kept[b]
        for kvh in (2, 7):
            pool = np.zeros((pages, 1, 1664), np.uint8)
            oracle.quantize_append(k_seq[:, kvh:kvh + 1], v_seq[:, kvh:kvh + 1], np.arange(n, dtype=np.int64), pool)
            got = cache[torch.from_numpy(bt[b, :pages].astype(np.int64)).to(dev), kvh].cpu().numpy()
            assert np.array_equal(got, pool[:, 0]), f"codes differ: seq {b} head {kvh}"
            qh = q.cpu().numpy()[b, kvh * w.gqa:(kvh + 1) * w.gqa][None]
            ref = oracle.decode_attention(pool, np.arange(pages, dtype=np.int32)[None], np.array([n]), qh, SCALE)[0]
            err = np.max(np.abs(out[b, kvh * w.gqa:(kvh + 1) * w.gqa] - ref))
            log(f"  seq {b} kv {kvh}: err {err:.2e}")
            assert err <= TOL


@pytest.mark.parametrize("fmt", PRESET_FMTS)
def test_preset_workload_qwen3_32b_16k_sampled(dev, fmt):
    """Qwen3-32B shape (8 x 16384 cached tokens + 1 appended, 64 q / 8 KV
    heads) in the benchmark's launch configuration: bulk fill, then the fused
    append + decode step; 2 sequences x 2 KV heads checked against the oracle
    (codes of all 16385 tokens, attention of the 8 query heads)."""
    w = inp.workload("qwen3_32b_16k")
    kf = _kfmt(fmt)
    region = oracle.region_bytes(fmt)
    log(f"preset qwen3_32b_16k fmt={fmt}: fill")
    bt, num_pages = inp.page_table(w)
    ctx = w.context
    cache = torch.zeros((num_pages, w.num_kv_heads, region), dtype=torch.uint8, device=dev)
    keep = (2, 7)
    kept = {}
    new_k, new_v = [], []
    for b in range(w.num_seqs):
        k, v = inp.sequence_kv(w, b, 0, ctx + 1, device=dev)
        gpu_append(k[:ctx], v[:ctx], torch.from_numpy(inp.slot_mapping(bt, b, 0, ctx)).to(dev), cache, fmt=kf)
        new_k.append(k[ctx:])
        new_v.append(v[ctx:])
        if b in keep:
            kept[b] = (k.cpu().numpy(), v.cpu().numpy())
        del k, v
    nk, nv = torch.cat(new_k).contiguous(), torch.cat(new_v).contiguous()
    q = inp.queries(w)
    lens = torch.full((w.num_seqs,), ctx + 1, dtype=torch.int32, device=dev)
    log(f"preset qwen3_32b_16k fmt={fmt}: fused append + decode")
    out = kvq.append_decode_attention(nk, nv, q.to(dev), cache, torch.from_numpy(bt).to(dev), lens, ctx + 1,
                                      out_dtype=torch.float16, fmt=kf).float().cpu().numpy()
    n = ctx + 1
    pages = int(math.ceil(n / 16))
    for b in keep:
        k_seq, v_seq = kept[b]
        for kvh in (1, 6):
            pool = np.zeros((pages, 1, region), np.uint8)
            oracle.quantize_append(k_seq[:, kvh:kvh + 1], v_seq[:, kvh:kvh + 1], np.arange(n, dtype=np.int64), pool,
                                   fmt=fmt)
            ids = torch.from_numpy(bt[b, :pages].astype(np.int64)).to(dev)
            got = cache[ids, kvh].cpu().numpy()
            assert np.array_equal(got, pool[:, 0]), f"codes differ: seq {b} head {kvh}"
            qh = q.numpy()[b, kvh * w.gqa:(kvh + 1) * w.gqa][None]
            ref = oracle.decode_attention(pool, np.arange(pages, dtype=np.int32)[None], np.array([n]), qh, SCALE,
                                          fmt=fmt)[0]
            err = np.max(np.abs(out[b, kvh * w.gqa:(kvh + 1) * w.gqa] - ref))
            log(f"  seq {b} kv {kvh}: err {err:.2e}")
            assert err <= TOL


def test_mixed_widths_recent_k8v4_history_k4v2(dev):
    """Two quantised caches of different widths in one step (older tokens in
    K4V2, the recent ones in k8v4): their partials share one workspace row
    and one combine, and equal the oracle's attention over the union."""
    B, Hq, Hkv = 3, 16, 2
    G = Hq // Hkv
    hist, recent = [700, 1, 130], [64, 17, 1]
    log(f"mixed widths hist={hist} recent={recent}")
    cache_h, pool_h, bt_h, _, q = _build_case(dev, B, Hq, Hkv, hist, seed=77)
    cache_r, pool_r, bt_r, _, _ = _build_case(dev, B, Hq, Hkv, recent, seed=78, fmt=(8, 4))
    f84 = _kfmt((8, 4))
    qd = torch.from_numpy(q).to(dev)
    Lh, Lr = max(hist), max(recent)
    s_h = kvq.decode_split_slots(B, Hq, Hkv, Lh, pages_per_split=4)
    s_r = kvq.decode_split_slots(B, Hq, Hkv, Lr, fmt=f84)
    total = s_h + s_r
    ws = torch.full((kvq.slots_workspace_bytes(B, Hq, total),), 0xFF, dtype=torch.uint8, device=dev)
    kvq.decode_partials_slots(qd, cache_r, torch.from_numpy(bt_r).to(dev),
                              torch.tensor(recent, dtype=torch.int32, device=dev), Lr, ws, 0, total, fmt=f84)
    kvq.decode_partials_slots(qd, cache_h, torch.from_numpy(bt_h).to(dev),
                              torch.tensor(hist, dtype=torch.int32, device=dev), Lh, ws, s_r, total,
                              pages_per_split=4)
    out = kvq.decode_combine_slots(ws, B, Hq, total).cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            kv = [oracle.dequant_slot(pool_h[bt_h[b, t // 16], h], t % 16) for t in range(hist[b])]
            kv += [oracle.dequant_slot(pool_r[bt_r[b, t // 16], h], t % 16, fmt=(8, 4)) for t in range(recent[b])]
            k_all = np.stack([x[0] for x in kv])
            v_all = np.stack([x[1] for x in kv])
            ref = oracle.attention_f64(k_all, v_all, q[b, h * G:(h + 1) * G], SCALE)
            err = np.max(np.abs(out[b, h * G:(h + 1) * G] - ref))
            assert err <= TOL, f"b={b} h={h} err={err}"


# --------------------------------------------------------------------------
# Several query rows per sequence (causal)
# --------------------------------------------------------------------------

MQ_CASES = [
    # B, Hq, Hkv, lens, q_len, pages_per_split, fmt
    (2, 8, 1, [40, 16], 2, 0, (4, 2)),        # G = 8: 16 (row, head) pairs, two column groups
    (3, 2, 2, [100, 8, 33], 8, 0, (4, 2)),     # G = 1: 8 rows fill one column group
    (2, 8, 2, [300, 47], 4, 2, (4, 2)),        # masked tokens straddle two splits of one page pair
    (1, 4, 4, [16], 16, 0, (4, 2)),            # q_len = whole sequence
    (2, 48, 3, [129, 64], 3, 4, (4, 2)),       # G = 16: 48 pairs per KV head
    (2, 8, 2, [513, 31], 5, 0, (8, 4)),
    (2, 4, 1, [77, 200], 6, 2, (4, 4)),
    (2, 4, 1, [34, 66], 5, 0, (4, 2)),         # two masked page pairs in one split
    (2, 16, 2, [200, 45], 4, 0, (3, 3)),
]


@pytest.mark.parametrize("B,Hq,Hkv,lens,M,pps,fmt", MQ_CASES)
def test_multi_query_decode_matches_oracle(dev, B, Hq, Hkv, lens, M, pps, fmt):
    log(f"multi-query B={B} Hq={Hq} Hkv={Hkv} lens={lens} q_len={M} pps={pps} fmt={fmt}")
    cache, pool, bt, lens_np, _ = _build_case(dev, B, Hq, Hkv, lens, seed=M * 100 + sum(lens), fmt=fmt)
    rng = np.random.default_rng(M + sum(lens))
    q = (rng.standard_normal((B, M, Hq, D)) * 1.5).astype(np.float16)
    ref = oracle.decode_attention_mq(pool, bt, lens_np, q, SCALE, fmt=fmt)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    kf = _kfmt(fmt)
    out = kvq.decode_attention_mq(qd, cache, btd, ld, L, pages_per_split=pps, fmt=kf).cpu().numpy()
    err = np.max(np.abs(out - ref))
    assert err <= TOL, f"err={err}"
    out16 = kvq.decode_attention_mq(qd, cache, btd, ld, L, out_dtype=torch.float16, pages_per_split=pps,
                                    fmt=kf).float().cpu().numpy()
    assert np.max(np.abs(out16 - ref)) <= TOL
    # q_len = 1 is the plain decode, bit for bit
    one = kvq.decode_attention_mq(qd[:, -1:].contiguous(), cache, btd, ld, L, pages_per_split=pps, fmt=kf)
    plain = kvq.decode_attention(qd[:, -1].contiguous(), cache, btd, ld, L, pages_per_split=pps, fmt=kf)
    assert torch.equal(one[:, 0], plain)


# --------------------------------------------------------------------------
# Pages of 32, 64 and 128 tokens
# --------------------------------------------------------------------------

def _build_case_paged(dev, B, Hq, Hkv, lens, seed, P, fmt=(4, 2), append_last=True):
    """Pool of P-token pages, the first lens[b] (or lens[b] - 1) tokens of every
    sequence appended on the GPU and by the oracle."""
    rng = np.random.default_rng(seed)
    kf = kvq.format_from_string(f"k{fmt[0]}v{fmt[1]}_g128", page_tokens=P)
    pb = kvq.page_bytes(kf)
    pages = [-(-n // P) for n in lens]
    N = sum(pages) + 2
    perm = rng.permutation(N)
    bt = np.full((B, max(pages) + 1), -1, np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    cache = torch.full((N, Hkv, pb), 0xFF, dtype=torch.uint8, device=dev)
    pool = np.full((N, Hkv, pb), 0xFF, np.uint8)
    kv = []
    for b, n in enumerate(lens):
        k = (rng.standard_normal((n, Hkv, D)) * rng.choice([0.5, 2])).astype(np.float16)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        k[:, :, rng.integers(0, D, 3)] *= 10
        kv.append((k, v))
        m = n if append_last else n - 1
        if m > 0:
            t = np.arange(m)
            slots = bt[b, t // P].astype(np.int64) * P + t % P
            gpu_append(torch.from_numpy(k[:m]).to(dev), torch.from_numpy(v[:m]).to(dev),
                       torch.from_numpy(slots).to(dev), cache, fmt=kf)
            oracle.quantize_append(k[:m], v[:m], slots, pool, fmt=fmt, page_tokens=P)
    q = (rng.standard_normal((B, Hq, D)) * 1.5).astype(np.float16)
    return cache, pool, bt, kv, q, kf


@pytest.mark.parametrize("P,fmt,B,Hq,Hkv,lens", [
    (32, (4, 2), 3, 8, 1, [100, 1, 257]),
    (64, (4, 2), 2, 64, 8, [513, 77]),
    (128, (8, 4), 2, 16, 2, [1000, 129]),
    (64, (4, 4), 4, 12, 4, [64, 65, 127, 300]),
    (32, (3, 3), 2, 16, 2, [333, 48]),
])
def test_paged_decode_matches_oracle(dev, P, fmt, B, Hq, Hkv, lens):
    log(f"paged decode P={P} fmt={fmt} B={B} Hq={Hq} Hkv={Hkv} lens={lens}")
    cache, pool, bt, _, q, kf = _build_case_paged(dev, B, Hq, Hkv, lens, seed=P + sum(lens), P=P, fmt=fmt)
    assert np.array_equal(cache.cpu().numpy(), pool)
    lens_np = np.asarray(lens, np.int64)
    ref = oracle.decode_attention(pool, bt, lens_np, q, SCALE, fmt=fmt, page_tokens=P)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    for pps in (0, 2, 6):            # splits of 2 or 6 regions cut pages of 32+ tokens
        out = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=pps, fmt=kf).cpu().numpy()
        err = np.max(np.abs(out - ref))
        assert err <= TOL, f"pps={pps} err={err}"
    # several query rows on the same pool
    M = 3
    qm = (np.random.default_rng(P).standard_normal((B, M, Hq, D))).astype(np.float16)
    refm = oracle.decode_attention_mq(pool, bt, lens_np, qm, SCALE, fmt=fmt, page_tokens=P)
    outm = kvq.decode_attention_mq(torch.from_numpy(qm).to(dev), cache, btd, ld, L, fmt=kf).cpu().numpy()
    assert np.max(np.abs(outm - refm)) <= TOL


@pytest.mark.parametrize("P,H,T,seed", [(32, 3, 300, 1), (128, 8, 8200, 2), (64, 8, 9000, 3)])
def test_paged_append_bit_exact(dev, P, H, T, seed):
    """Both append kernels (the last two cases select the one-lane-per-group
    kernel) at page sizes above 16, with skipped and out-of-pool slots."""
    rng = np.random.default_rng(500 + seed)
    log(f"paged append P={P} H={H} T={T}")
    fmt = (4, 2) if seed != 3 else (8, 4)
    kf = kvq.format_from_string(f"k{fmt[0]}v{fmt[1]}_g128", page_tokens=P)
    pb = kvq.page_bytes(kf)
    N = -(-T // P) + 3
    k = _mixed_tokens(rng, T, H)
    v = _mixed_tokens(rng, T, H)
    slots = rng.permutation(N * P)[:T].astype(np.int64)
    slots[rng.integers(0, T, 5)] = -1
    slots[0] = N * P + 3
    cache = torch.full((N, H, pb), 0x3C, dtype=torch.uint8, device=dev)
    gpu_append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), torch.from_numpy(slots).to(dev), cache,
               fmt=kf)
    pool = np.full((N, H, pb), 0x3C, np.uint8)
    ok = (slots >= 0) & (slots < N * P)
    oracle.quantize_append(k[ok], v[ok], slots[ok], pool, fmt=fmt, page_tokens=P)
    diff = np.argwhere(cache.cpu().numpy() != pool)
    assert diff.size == 0, f"{len(diff)} bytes differ, first at {diff[:5].tolist()}"


@pytest.mark.parametrize("P,pps", [(64, 0), (32, 2), (128, 4)])
def test_paged_fused_append_decode(dev, P, pps):
    B, Hq, Hkv, lens = 3, 16, 2, [400, 33, 777]
    log(f"paged fused append P={P} pps={pps}")
    cache, pool, bt, kv, q, kf = _build_case_paged(dev, B, Hq, Hkv, lens, seed=P * 3 + pps, P=P,
                                                   append_last=False)
    new_k = np.stack([kv[b][0][n - 1] for b, n in enumerate(lens)])
    new_v = np.stack([kv[b][1][n - 1] for b, n in enumerate(lens)])
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = kvq.append_decode_attention(torch.from_numpy(new_k).to(dev), torch.from_numpy(new_v).to(dev), qd, cache,
                                      btd, ld, max(lens), pages_per_split=pps, fmt=kf).cpu().numpy()
    last = np.array([bt[b, (n - 1) // P] * P + (n - 1) % P for b, n in enumerate(lens)], np.int64)
    oracle.quantize_append(new_k, new_v, last, pool, page_tokens=P)
    assert np.array_equal(cache.cpu().numpy(), pool)
    ref = oracle.decode_attention(pool, bt, np.asarray(lens), q, SCALE, page_tokens=P)
    assert np.max(np.abs(out - ref)) <= TOL


def test_pool_beyond_4_gib(dev):
    """Page ids whose byte offsets exceed 2^32 (a 4.4 GB pool of 8-head
    pages): append and decode address them with 64-bit arithmetic.  Only a
    few pages at the top of the pool are used; the oracle gets them
    relabelled to a small pool."""
    Hkv, Hq, B = 8, 64, 2
    num_pages = (5 << 30) // (Hkv * 1664)               # ~5 GiB
    lens = [100, 37]
    rng = np.random.default_rng(4096)
    log(f"pool beyond 4 GiB: {num_pages} pages")
    cache = torch.empty((num_pages, Hkv, 1664), dtype=torch.uint8, device=dev)
    top = np.arange(num_pages - 12, num_pages, dtype=np.int32)
    rng.shuffle(top)
    pages = [-(-n // 16) for n in lens]
    bt = np.full((B, max(pages)), -1, np.int32)
    bt[0, :pages[0]] = top[:pages[0]]
    bt[1, :pages[1]] = top[pages[0]:pages[0] + pages[1]]
    assert int(bt.max()) * Hkv * 1664 > (1 << 32)
    small = {int(p): i for i, p in enumerate(top)}
    bt_small = np.vectorize(lambda p: small.get(int(p), -1))(bt).astype(np.int32)
    pool = np.zeros((len(top), Hkv, 1664), np.uint8)
    for b, n in enumerate(lens):
        k = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        gpu_append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                   torch.from_numpy(inp.slot_mapping(bt, b, 0, n)).to(dev), cache)
        oracle.quantize_append(k, v, inp.slot_mapping(bt_small, b, 0, n), pool)
    got = cache[torch.from_numpy(top.astype(np.int64)).to(dev)].cpu().numpy()
    used = np.zeros(len(top), bool)
    used[[small[int(p)] for p in bt[bt >= 0]]] = True
    for i in np.nonzero(used)[0]:
        r = 0
        # compare the written token slots only (the rest of the pool is uninitialised)
        b = 0 if top[i] in bt[0] else 1
        j = list(bt[b]).index(top[i])
        r = min(16, lens[b] - 16 * j)
        m = valid_byte_mask(r)
        assert np.array_equal(got[i][:, m], pool[i][:, m])
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    out = kvq.decode_attention(torch.from_numpy(q).to(dev), cache, torch.from_numpy(bt).to(dev),
                               torch.tensor(lens, dtype=torch.int32, device=dev), max(lens)).cpu().numpy()
    ref = oracle.decode_attention(pool, bt_small, np.array(lens), q, SCALE)
    assert np.max(np.abs(out - ref)) <= TOL
    del cache
    torch.cuda.empty_cache()


def test_checkpoint_and_resume(dev):
    """The cache state is the caller's byte pool plus block tables: a pool
    dumped to host memory and loaded into a fresh device buffer decodes to the
    same bits, and keeps accepting appends exactly as the original."""
    B, Hq, Hkv, lens = 2, 16, 2, [300, 77]
    cache, pool, bt, lens_np, q = _build_case(dev, B, Hq, Hkv, lens, seed=31)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    before = kvq.decode_attention(qd, cache, btd, ld, max(lens)).cpu()
    host = cache.cpu().numpy().copy()                       # checkpoint
    restored = torch.from_numpy(host).to(dev)               # resume into a new buffer
    assert torch.equal(kvq.decode_attention(qd, restored, btd, ld, max(lens)).cpu(), before)
    # one more token per sequence into both: identical bytes
    rng = np.random.default_rng(32)
    kn = torch.from_numpy(rng.standard_normal((B, Hkv, D)).astype(np.float16)).to(dev)
    vn = torch.from_numpy(rng.standard_normal((B, Hkv, D)).astype(np.float16)).to(dev)
    slots = torch.tensor([int(bt[b, n // 16]) * 16 + n % 16 for b, n in enumerate(lens)], device=dev)
    gpu_append(kn, vn, slots, cache)
    gpu_append(kn, vn, slots, restored)
    assert torch.equal(cache.cpu(), restored.cpu())
