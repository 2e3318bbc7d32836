"""GPU parity of the page-balanced key preset ("k4v2_g128_pb"): the HIP
whole-page append and the decode through the C ABI against the oracle
(kvqo_quantize_append_pb, kvqo_decode_attention_pb).

Bar: pool bytes bit-identical to the oracle's (codes, metadata and column
scales; slots the call does not fill keep their bytes); attention max-abs
error <= 2e-3 against the oracle's fp64 attention over the same bytes.
"""
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
REGION = 1792


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvq.load()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def pb():
    return kvq.format_from_string("kvarn_k4v2_g128_pb")


def log(msg):
    print(msg, flush=True)


def _hadamard():
    h = np.array([[1.0]])
    while h.shape[0] < D:
        h = np.block([[h, h], [h, -h]])
    return h


HM = _hadamard()


def _unbalanced_keys(rng, T, H):
    """fp16 keys [T][H][128] whose rotated channels have very different
    scales within a page (factors 2^-7 .. 2^7, fixed per (block, head)), so
    that the column exponents take values across [-6, 6]; x = H y / 128."""
    x = np.empty((T, H, D))
    for b0 in range(0, T, 16):
        for h in range(H):
            col = 2.0 ** rng.integers(-7, 8, D)
            y = rng.standard_normal((min(16, T - b0), D)) * col
            x[b0:b0 + 16, h] = y @ HM / 128.0
    return x.astype(np.float16)


def _regime_keys(rng, T, H):
    """fp16 rows of several regimes: normal, fp16 subnormals, large, outlier
    channels, zero rows, a constant rotation, Student-t."""
    x = np.empty((T, H, D))
    kinds = rng.integers(0, 7, (T, H))
    for t in range(T):
        for h in range(H):
            k = kinds[t, h]
            if k == 0:
                r = rng.standard_normal(D)
            elif k == 1:
                r = rng.standard_normal(D) * 1e-5
            elif k == 2:
                r = rng.standard_normal(D) * 300.0
            elif k == 3:
                r = rng.standard_normal(D)
                r[rng.integers(0, D, 4)] *= 30.0
            elif k == 4:
                r = np.zeros(D)
            elif k == 5:
                r = np.zeros(D)
                r[0] = rng.choice([-3.0, 0.5, 7.25])
            else:
                r = rng.standard_t(3, D)
            x[t, h] = r
    return x.astype(np.float16)


def _block_slots(rng, T, num_pages):
    """Slots of T call tokens in whole-page blocks of 16, each block on its own
    random page (fewer pages than the pool holds)."""
    nb = -(-T // 16)
    pages = rng.permutation(num_pages)[:nb]
    t = np.arange(T)
    return (pages[t // 16] * 16 + t % 16).astype(np.int64)


def _append_both(dev, pb, k, v, slots, num_pages, fill=0x3C, kstride_pad=0):
    T, H, _ = k.shape
    if kstride_pad:
        kb = torch.zeros((T, H + kstride_pad, D), dtype=torch.float16)
        vb = torch.zeros((T, H + kstride_pad, D), dtype=torch.float16)
        kb[:, :H] = torch.from_numpy(k)
        vb[:, :H] = torch.from_numpy(v)
        kd, vd = kb.to(dev)[:, :H], vb.to(dev)[:, :H]
    else:
        kd, vd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    cache = torch.full((num_pages, H, REGION), fill, dtype=torch.uint8, device=dev)
    kvq.quantize_append(kd, vd, torch.from_numpy(slots).to(dev), cache, fmt=pb)
    pool = np.full((num_pages, H, REGION), fill, np.uint8)
    oracle.quantize_append_pb(k, v, slots, pool)
    return cache, pool


def _assert_same(got, want):
    diff = np.argwhere(got != want)
    assert diff.size == 0, f"{len(diff)} bytes differ, first at {diff[:5].tolist()}"


def test_pb_format(dev, pb):
    assert pb.k_bits == 4 and pb.v_bits == 2 and pb.block_size == 16 and pb.key_norm == kvq.KEY_NORM_PAGE
    assert kvq.page_bytes(pb) == REGION == oracle.PB_REGION


@pytest.mark.parametrize("H,T,num_pages,seed,kind", [
    (1, 16, 2, 1, "unbalanced"), (1, 37, 8, 2, "unbalanced"), (3, 100, 12, 3, "regimes"),
    (8, 515, 40, 4, "unbalanced"), (8, 8200, 600, 5, "regimes"), (2, 4096, 300, 6, "unbalanced")])
def test_pb_append_bit_exact(dev, pb, H, T, num_pages, seed, kind):
    rng = np.random.default_rng(500 + seed)
    log(f"pb append H={H} T={T} pages={num_pages} {kind}")
    k = (_unbalanced_keys if kind == "unbalanced" else _regime_keys)(rng, T, H)
    v = _regime_keys(rng, T, H)
    slots = _block_slots(rng, T, num_pages)
    cache, pool = _append_both(dev, pb, k, v, slots, num_pages, kstride_pad=seed % 2)
    _assert_same(cache.cpu().numpy(), pool)
    # the column exponents are not all zero on unbalanced keys
    if kind == "unbalanced":
        used = pool[np.unique(slots // 16)][:, :, 1664:]
        assert len(np.unique(used)) > 3


def test_pb_append_holes_and_skipped_blocks(dev, pb):
    """Absent rows (negative slots, a slot off its block's run), a ragged last
    block, and blocks that are skipped: a negative first slot, a first slot
    that is not a page start, a page outside the pool."""
    rng = np.random.default_rng(77)
    H, T, num_pages = 2, 16 * 7 + 5, 12
    k = _unbalanced_keys(rng, T, H)
    v = _regime_keys(rng, T, H)
    slots = _block_slots(rng, T, num_pages)
    slots[3] = -1                       # absent row of block 0
    slots[16 + 9] = slots[16 + 9] + 1   # off the run: absent (its slot is another row's)
    slots[16 + 10] = -1
    slots[32] = -1                      # block 2 skipped: negative first slot
    slots[48] += 1                      # block 3 skipped: not a page start
    slots[64:80] = num_pages * 16 + np.arange(16)   # block 4 skipped: outside the pool
    cache, pool = _append_both(dev, pb, k, v, slots, num_pages, fill=0xA5)
    _assert_same(cache.cpu().numpy(), pool)


def test_pb_append_zero_block_and_subnormal_rows(dev, pb):
    """An all-zero page (every column zero: exponent -6 everywhere), a page of
    fp16 subnormal keys, and a page with one non-zero row."""
    rng = np.random.default_rng(9)
    H, T, num_pages = 1, 48, 4
    k = np.zeros((T, H, D), np.float16)
    k[16:32] = (rng.standard_normal((16, H, D)) * 3e-6).astype(np.float16)
    k[40] = rng.standard_normal((H, D)).astype(np.float16)
    v = _regime_keys(rng, T, H)
    slots = np.arange(T, dtype=np.int64)
    cache, pool = _append_both(dev, pb, k, v, slots, num_pages)
    _assert_same(cache.cpu().numpy(), pool)
    assert np.all(pool[0, 0, 1664:] == (15 - 6) * 4)


def _build_pb_case(dev, pb, B, Hq, Hkv, lens, seed):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int64)
    pages = [max(1, int(math.ceil(n / 16))) for n in lens]
    num_pages = sum(pages) + 3
    perm = rng.permutation(num_pages)
    bt = np.full((B, max(pages) + 2), -1, np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    cache = torch.full((num_pages, Hkv, REGION), 0xFF, dtype=torch.uint8, device=dev)
    pool = np.full((num_pages, Hkv, REGION), 0xFF, np.uint8)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        k = _unbalanced_keys(rng, n, Hkv)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        slots = inp.slot_mapping(bt, b, 0, n)
        kvq.quantize_append(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev),
                            torch.from_numpy(slots).to(dev), cache, fmt=pb)
        oracle.quantize_append_pb(k, v, slots, pool)
    q = (rng.standard_normal((B, Hq, D)) * rng.choice([0.5, 1, 3])).astype(np.float16)
    return cache, pool, bt, lens, q


PB_DECODE = [
    # B, Hq, Hkv, lens
    (1, 1, 1, [1]),
    (1, 8, 1, [15]),
    (1, 8, 1, [16]),
    (2, 4, 1, [17, 33]),
    (2, 16, 2, [100, 31]),
    (3, 64, 8, [300, 1, 257]),
    (1, 32, 2, [700]),              # 16 query heads per KV head: two head groups
    (4, 12, 4, [64, 65, 127, 300]),
    (2, 8, 1, [0, 50]),             # an empty sequence
]


@pytest.mark.parametrize("B,Hq,Hkv,lens", PB_DECODE)
def test_pb_decode_matches_oracle(dev, pb, B, Hq, Hkv, lens):
    log(f"pb decode B={B} Hq={Hq} Hkv={Hkv} lens={lens}")
    cache, pool, bt, lens_np, q = _build_pb_case(dev, pb, B, Hq, Hkv, lens, seed=B * 100 + Hq + sum(lens))
    _assert_same(cache.cpu().numpy(), pool)
    ref = oracle.decode_attention_pb(pool, bt, lens_np, q, SCALE)
    qd = torch.from_numpy(q).to(dev)
    btd = torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = max(1, int(lens_np.max()))
    for pps in (0, 2, 6):
        out = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=pps, fmt=pb)
        err = np.max(np.abs(out.cpu().numpy() - ref))
        assert err <= TOL, f"pps={pps} err={err}"
    out16 = kvq.decode_attention(qd, cache, btd, ld, L, out_dtype=torch.float16, fmt=pb)
    err16 = np.max(np.abs(out16.float().cpu().numpy() - ref))
    assert err16 <= TOL, f"fp16 out err={err16}"


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (32, 2)])
def test_pb_decode_pair_loop_lengths_match_oracle(dev, pb, Hq, Hkv):
    # waves of 4 to 16 page pairs per split at 128 and 64 pages per split: the
    # unguarded rounds of three pairs, every length of the guarded last stretch
    # and a masked last pair (two head groups: the guarded loop throughout)
    lens = [600, 700, 800, 900, 1000, 1100, 1300, 2049, 4000]
    B = len(lens)
    log(f"pb decode pair-loop lengths Hq={Hq} Hkv={Hkv}")
    cache, pool, bt, lens_np, q = _build_pb_case(dev, pb, B, Hq, Hkv, lens, seed=7001 + Hq)
    _assert_same(cache.cpu().numpy(), pool)
    ref = oracle.decode_attention_pb(pool, bt, lens_np, q, SCALE)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    for pps in (128, 64, 0):
        out = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=pps, fmt=pb)
        err = np.max(np.abs(out.cpu().numpy() - ref))
        assert err <= TOL, f"pps={pps} err={err}"


def test_pb_decode_two_phase_matches_one_call(dev, pb):
    cache, pool, bt, lens_np, q = _build_pb_case(dev, pb, 3, 16, 2, [400, 1, 777], seed=31)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    L = int(lens_np.max())
    one = kvq.decode_attention(qd, cache, btd, ld, L, pages_per_split=4, fmt=pb)
    ws = kvq.alloc_workspace(3, 16, 2, L, 4, device=dev, fmt=pb)
    kvq.decode_partials(qd, cache, btd, ld, L, ws, pages_per_split=4, fmt=pb)
    two = kvq.decode_combine(ws, ld, 16, 2, L, pages_per_split=4, fmt=pb)
    assert torch.equal(one, two)


def test_pb_unsupported_calls(dev, pb):
    cache, pool, bt, lens_np, q = _build_pb_case(dev, pb, 1, 8, 1, [40], seed=5)
    qd, btd = torch.from_numpy(q).to(dev), torch.from_numpy(bt).to(dev)
    ld = torch.from_numpy(lens_np.astype(np.int32)).to(dev)
    nk = torch.zeros((1, 1, D), dtype=torch.float16, device=dev)
    with pytest.raises(kvq.KvqError, match="UNSUPPORTED"):
        kvq.append_decode_attention(nk, nk, qd, cache, btd, ld, 40, fmt=pb)
    with pytest.raises(kvq.KvqError, match="UNSUPPORTED"):
        kvq.decode_attention_mq(torch.zeros((1, 2, 8, D), dtype=torch.float16, device=dev), cache, btd, ld, 40,
                                fmt=pb)
    # nothing was written
    _assert_same(cache.cpu().numpy(), pool)


def test_pb_workload_qwen3_32b_16k_sampled(dev, pb):
    """The benchmark's workload shape with page-balanced keys: 8 x 16385
    tokens appended on the GPU in one call per sequence, decode in the
    heuristic split; 2 sequences x 2 KV heads against the oracle (all pages'
    bytes, attention of their 8 query heads)."""
    w = inp.workload("qwen3_32b_16k")
    bt, num_pages = inp.page_table(w)
    n = w.context + 1
    log("pb qwen3_32b_16k: fill")
    cache = torch.zeros((num_pages, w.num_kv_heads, REGION), dtype=torch.uint8, device=dev)
    keep = (1, 6)
    kept = {}
    for b in range(w.num_seqs):
        k, v = inp.sequence_kv(w, b, 0, n, device=dev)
        kvq.quantize_append(k, v, torch.from_numpy(inp.slot_mapping(bt, b, 0, n)).to(dev), cache, fmt=pb)
        if b in keep:
            kept[b] = (k.cpu().numpy(), v.cpu().numpy())
        del k, v
    q = inp.queries(w)
    lens = torch.full((w.num_seqs,), n, dtype=torch.int32, device=dev)
    log("pb qwen3_32b_16k: decode")
    out = kvq.decode_attention(q.to(dev), cache, torch.from_numpy(bt).to(dev), lens, n, fmt=pb).cpu().numpy()
    pages = int(math.ceil(n / 16))
    for b in keep:
        k_seq, v_seq = kept[b]
        for kvh in (0, 5):
            pool = np.zeros((pages, 1, REGION), np.uint8)
            oracle.quantize_append_pb(np.ascontiguousarray(k_seq[:, kvh:kvh + 1]),
                                      np.ascontiguousarray(v_seq[:, kvh:kvh + 1]),
                                      np.arange(n, dtype=np.int64), pool)
            ids = torch.from_numpy(bt[b, :pages].astype(np.int64)).to(dev)
            got = cache[ids, kvh].cpu().numpy()
            # both pools start as zeros, so the last page's unfilled slots agree too
            assert np.array_equal(got, pool[:, 0]), f"bytes differ: seq {b} head {kvh}"
            qh = q.numpy()[b, kvh * w.gqa:(kvh + 1) * w.gqa][None]
            ref = oracle.decode_attention_pb(pool, np.arange(pages, dtype=np.int32)[None], np.array([n]), qh,
                                             SCALE)[0]
            err = np.max(np.abs(out[b, kvh * w.gqa:(kvh + 1) * w.gqa] - ref))
            log(f"  seq {b} kv {kvh}: err {err:.2e}")
            assert err <= TOL


@pytest.mark.parametrize("sink,window,hist", [(4, 44, [300, 1000, 0]), (0, 16, [512, 80, 16])])
def test_pb_history_with_fp16_window(dev, pb, sink, window, hist):
    """The serving layout for page-balanced keys: whole pages of history in
    the page-balanced cache, the sink and the recent (partly filled) page's
    tokens uncompressed in an fp16 cache; both caches' partials merged by one
    combine equal the oracle's attention over the union (history dequantised
    by kvqo_dequant_slot_pb, window raw)."""
    B, Hq, Hkv = len(hist), 16, 2
    G = Hq // Hkv
    log(f"pb history sink={sink} window={window} hist={hist}")
    rng = np.random.default_rng(sink * 7 + window + sum(hist))
    cache_h, pool_h, bt_h, lens_h, q = _build_pb_case(dev, pb, B, Hq, Hkv, hist, seed=sum(hist) + 11)
    f16 = kvq.format_from_string("fp16")
    nf = sink + window
    pages_f = -(-max(nf, 1) // 16)
    bt_f = np.arange(B * pages_f, dtype=np.int32).reshape(B, pages_f)
    cache_f = torch.full((B * pages_f, Hkv, 8192), 0xFF, dtype=torch.uint8, device=dev)
    kf = (rng.standard_normal((B, nf, Hkv, D)) * 0.8).astype(np.float16)
    vf = rng.standard_normal((B, nf, Hkv, D)).astype(np.float16)
    for b in range(B):
        kvq.quantize_append(torch.from_numpy(kf[b]).to(dev), torch.from_numpy(vf[b]).to(dev),
                            torch.from_numpy(inp.slot_mapping(bt_f, b, 0, nf)).to(dev), cache_f, fmt=f16)
    qd = torch.from_numpy(q).to(dev)
    Lh, Lf = max(int(lens_h.max()), 1), max(nf, 1)
    s_h = kvq.decode_split_slots(B, Hq, Hkv, Lh, fmt=pb)
    s_f = kvq.decode_split_slots(B, Hq, Hkv, Lf, fmt=f16)
    total = s_h + s_f
    ws = torch.full((kvq.slots_workspace_bytes(B, Hq, total),), 0xFF, dtype=torch.uint8, device=dev)
    kvq.decode_partials_slots(qd, cache_h, torch.from_numpy(bt_h).to(dev),
                              torch.from_numpy(lens_h.astype(np.int32)).to(dev), Lh, ws, 0, total, fmt=pb)
    kvq.decode_partials_slots(qd, cache_f, torch.from_numpy(bt_f).to(dev),
                              torch.full((B,), nf, dtype=torch.int32, device=dev), Lf, ws, s_h, total,
                              rotated=True, fmt=f16)
    out = kvq.decode_combine_slots(ws, B, Hq, total).cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            kh = np.zeros((hist[b], D)); vh = np.zeros((hist[b], D))
            for t in range(hist[b]):
                kh[t], vh[t] = oracle.dequant_slot_pb(np.ascontiguousarray(pool_h[bt_h[b, t // 16], h]), t % 16)
            k_all = np.concatenate([kf[b, :, h].astype(np.float64), kh])
            v_all = np.concatenate([vf[b, :, h].astype(np.float64), vh])
            ref = oracle.attention_f64(k_all, v_all, q[b, h * G:(h + 1) * G], SCALE)
            err = np.max(np.abs(out[b, h * G:(h + 1) * G] - ref))
            assert err <= TOL, f"b={b} h={h} err={err}"
