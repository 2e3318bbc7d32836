"""kvq_append_decode_attention_noalloc against kvq_append_decode_attention
(GPU, through the C ABI).

The no-alloc entry point is the fused append-and-decode step with its split
partials in the library's fixed per-device array instead of a caller
workspace.  Two calls in a row -- the second smaller, so that it runs over
what the first left in the array -- must give the cache bytes and the output
of the workspace entry point on the same inputs, bit for bit, and both must
match the oracle."""
import ctypes
import math

import numpy as np
import pytest
import torch

import kvq_inputs as inp
import oracle
import quantized_decode_attention_quantize_amd as kvq

D = 128
SCALE = 1.0 / math.sqrt(D)
TOL = 2e-3


def _case(dev, rng, B, Hq, Hkv, lens):
    pages = [int(math.ceil(n / 16)) for n in lens]
    num_pages = sum(pages) + 1
    perm = rng.permutation(num_pages)
    bt = np.zeros((B, max(pages)), np.int32)
    o = 0
    for b, p in enumerate(pages):
        bt[b, :p] = perm[o:o + p]
        o += p
    cache = torch.zeros((num_pages, Hkv, 1664), dtype=torch.uint8, device=dev)
    pool = np.zeros((num_pages, Hkv, 1664), np.uint8)
    nk = np.zeros((B, Hkv, D), np.float16)
    nv = np.zeros((B, Hkv, D), np.float16)
    for b, n in enumerate(lens):
        k = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        v = rng.standard_normal((n, Hkv, D)).astype(np.float16)
        nk[b], nv[b] = k[n - 1], v[n - 1]
        slots = inp.slot_mapping(bt, b, 0, n - 1)
        if n > 1:
            kvq.quantize_append(torch.from_numpy(k[:n - 1]).to(dev), torch.from_numpy(v[:n - 1]).to(dev),
                                torch.from_numpy(slots).to(dev), cache)
        oracle.quantize_append(k, v, inp.slot_mapping(bt, b, 0, n), pool)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    return bt, cache, pool, nk, nv, q


@pytest.mark.gpu
def test_noalloc_step_matches_the_workspace_step_twice():
    dev = torch.device("cuda:0")
    lib = kvq.load()
    fmt = kvq.format_from_string("k4v2_g128")
    rng = np.random.default_rng(20260605 + 404)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    cases = [(8, 64, 8, list(rng.integers(2000, 4100, 8))), (3, 16, 2, [300, 17, 129])]
    for B, Hq, Hkv, lens in cases:
        lens = [int(n) for n in lens]
        print(f"noalloc: B={B} Hq={Hq} Hkv={Hkv} lens={lens}", flush=True)
        bt, cache, pool, nk, nv, q = _case(dev, rng, B, Hq, Hkv, lens)
        L = max(lens)
        assert kvq.decode_workspace_bytes(B, Hq, Hkv, L) <= kvq.NOALLOC_SCRATCH_BYTES
        btd, ld = torch.from_numpy(bt).to(dev), torch.tensor(lens, dtype=torch.int32, device=dev)
        qd, nkd, nvd = torch.from_numpy(q).to(dev), torch.from_numpy(nk).to(dev), torch.from_numpy(nv).to(dev)
        cache_ws = cache.clone()
        out_ws = kvq.append_decode_attention(nkd, nvd, qd, cache_ws, btd, ld, L, out_dtype=torch.float32)
        out_na = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.kvq_append_decode_attention_noalloc(
            ctypes.byref(fmt), P(out_na.data_ptr()), 1, P(nkd.data_ptr()), P(nvd.data_ptr()), i64(Hkv * D),
            i64(Hkv * D), P(qd.data_ptr()), P(cache.data_ptr()), i64(cache.shape[0]), P(btd.data_ptr()),
            i32(bt.shape[1]), P(ld.data_ptr()), i32(B), i32(Hq), i32(Hkv), i32(L), ctypes.c_float(SCALE), i32(0),
            P(stream))
        assert st == 0, kvq.load().kvq_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(cache.cpu(), cache_ws.cpu())
        assert torch.equal(out_na.cpu(), out_ws.cpu())
        assert np.array_equal(cache.cpu().numpy(), pool)
        ref = oracle.decode_attention(pool, bt, np.asarray(lens), q, SCALE)
        err = float(np.max(np.abs(out_na.cpu().numpy() - ref)))
        print(f"  bit-identical to the workspace call; oracle max-abs err {err:.2e}", flush=True)
        assert err <= TOL
    # the binding's wrapper marshals to the same call (fp16 output)
    B, Hq, Hkv, lens = 2, 8, 1, [40, 16]
    bt, cache, pool, nk, nv, q = _case(dev, rng, B, Hq, Hkv, lens)
    btd, ld = torch.from_numpy(bt).to(dev), torch.tensor(lens, dtype=torch.int32, device=dev)
    cache_ws = cache.clone()
    args = (torch.from_numpy(nk).to(dev), torch.from_numpy(nv).to(dev), torch.from_numpy(q).to(dev))
    o16 = kvq.append_decode_attention_noalloc(*args, cache, btd, ld, 40,
                                              torch.empty((B, Hq, D), dtype=torch.float16, device=dev),
                                              pages_per_split=2)
    w16 = kvq.append_decode_attention(*args, cache_ws, btd, ld, 40, out_dtype=torch.float16, pages_per_split=2)
    torch.cuda.synchronize()
    assert torch.equal(o16.cpu(), w16.cpu()) and torch.equal(cache.cpu(), cache_ws.cpu())
