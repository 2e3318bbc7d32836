"""The C-ABI library loads, exports every declared entry point, and validates
host-visible arguments without launching anything (CPU only)."""
import ctypes
import os
import re

import pytest
import torch

import quantized_decode_attention_quantize_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADER = os.path.join(INCLUDE, "kvq.h")


def header_texts():
    """Every public header (kvq.h and the measurement aids' kvq_measure.h)."""
    return {f: open(os.path.join(INCLUDE, f)).read() for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h")}


def declared_functions():
    names = set()
    for text in header_texts().values():
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = kvq.load()
    names = declared_functions()
    assert "kvq_quantize_append" in names and "kvq_decode_attention" in names
    for name in names:
        assert hasattr(lib, name), name


# every preset name the library accepts; the header must document each one
PRESETS = {"k4v2_g128": (4, 2), "k4v4_g128": (4, 4), "k8v2_g128": (8, 2), "k8v4_g128": (8, 4),
           "k3v3_g128": (3, 3)}


def test_header_documents_every_accepted_preset():
    """Each preset string the parser accepts (with and without the kvarn_
    prefix) appears in kvq.h's description of kvq_format_from_string, and
    the header's bit-width sentence names its key and value widths; a string
    the parser rejects is not presented as a preset there."""
    lib = kvq.load()
    text = open(HEADER).read()
    i = text.index("Parse a preset name")
    doc = text[i:text.index("kvq_status kvq_format_from_string", i)]
    f = kvq.Format()
    for name, (kb, vb) in PRESETS.items():
        for full in (name, "kvarn_" + name):
            assert lib.kvq_format_from_string(full.encode(), ctypes.byref(f)) == 0, full
            assert (f.k_bits, f.v_bits) == (kb, vb)
        assert f'"{name}"' in doc, name
        assert name in text[:text.index("#ifndef KVQ_H")], name
    assert '"kvarn_"' in doc
    assert lib.kvq_format_from_string(b"fp16", ctypes.byref(f)) == 0 and '"fp16"' in doc
    for quoted in re.findall(r'"([a-z0-9_]+)"', doc):
        if quoted == "kvarn_":
            continue
        assert lib.kvq_format_from_string(quoted.encode(), ctypes.byref(f)) == 0, quoted


def test_measurement_aids_live_in_their_own_header():
    """The timing hook and the read probes are declared in kvq_measure.h, not
    beside the decode path in kvq.h."""
    texts = header_texts()
    assert set(texts) >= {"kvq.h", "kvq_measure.h"}
    for name in ("kvq_set_split_kernel_events", "kvq_stream_read_probe", "kvq_page_walk_probe"):
        assert name + "(" in texts["kvq_measure.h"].replace(" (", "(")
        assert name not in texts["kvq.h"]


def test_format_and_sizes():
    lib = kvq.load()
    f = kvq.Format()
    assert lib.kvq_format_from_string(b"kvarn_k4v2_g128", ctypes.byref(f)) == 0
    assert (f.head_dim, f.group_size, f.k_bits, f.v_bits, f.block_size) == (128, 128, 4, 2, 16)
    assert lib.kvq_format_from_string(b"k4v2_g128", ctypes.byref(f)) == 0
    assert lib.kvq_format_from_string(b"k3v2_g128", ctypes.byref(f)) == 3
    assert lib.kvq_format_from_string(b"k4v2_g64", ctypes.byref(f)) == 3
    assert lib.kvq_format_from_string(None, ctypes.byref(f)) == 1
    assert kvq.page_bytes() == 1664 == 64 * 16 + 32 * 16 + 4 * 16 + 4 * 16
    # 104 bytes per token per KV head against 512 for fp16: 4.92x, inside the
    # 3-5x capacity range the KVarN pages report
    ratio = 512 / (1664 / 16)
    assert 3.0 <= ratio <= 5.0 and abs(ratio - 4.923) < 1e-3
    assert kvq.cache_bytes(10, 8) == 10 * 8 * 1664
    for bad in (kvq.Format(128, 128, 8, 8, 16), kvq.Format(128, 128, 2, 2, 16), kvq.Format(128, 64, 4, 2, 16),
                kvq.Format(128, 128, 3, 2, 16), kvq.Format(128, 128, 4, 3, 16), kvq.Format(128, 128, 3, 4, 16),
                kvq.Format(128, 128, 4, 2, 48), kvq.Format(128, 128, 4, 2, 256), kvq.Format(128, 128, 16, 16, 32)):
        assert lib.kvq_page_bytes(ctypes.byref(bad)) == 0
        assert lib.kvq_cache_bytes(ctypes.byref(bad), 10, 8) == 0


@pytest.mark.parametrize("preset,kb,vb", [("k4v4_g128", 4, 4), ("kvarn_k4v4_g128", 4, 4), ("k8v2_g128", 8, 2),
                                          ("k8v4_g128", 8, 4), ("kvarn_k8v4_g128", 8, 4), ("k3v3_g128", 3, 3),
                                          ("kvarn_k3v3_g128", 3, 3)])
def test_other_bit_width_presets(preset, kb, vb):
    """Presets of the same pipeline at other widths: region = key codes (16 x
    16 kb bytes) + value codes (16 x 16 vb) + two 16 x 4 metadata arrays."""
    f = kvq.format_from_string(preset)
    assert (f.head_dim, f.group_size, f.k_bits, f.v_bits, f.block_size) == (128, 128, kb, vb, 16)
    assert kvq.page_bytes(f) == 16 * (16 * kb + 16 * vb + 8)
    assert kvq.page_bytes(f) % 128 == 0
    assert kvq.cache_bytes(3, 8, f) == 3 * 8 * kvq.page_bytes(f)


def test_kv_memory_closed_form():
    """Sizing check of the bf16 cache figure on the HBM page (Llama-3.1-70B:
    80 layers, 8 KV heads, head_dim 128): 2*80*8*128*2 bytes per token, about
    0.31 MB, about 40 GiB at 128K tokens; the K4V2 pool is 4.92x smaller."""
    per_token_bf16 = 2 * 80 * 8 * 128 * 2
    assert per_token_bf16 == 327_680
    assert abs(per_token_bf16 * 131072 / 2 ** 30 - 40.0) < 1e-9
    k4v2 = kvq.cache_bytes(131072 // 16, 8) * 80
    assert abs(per_token_bf16 * 131072 / k4v2 - 512 / 104) < 1e-12


def test_workspace_sizing_and_heuristic():
    pps = kvq.decode_pages_per_split(8, 64, 8, 16385)
    assert pps > 0 and pps % 2 == 0
    n = kvq.decode_workspace_bytes(8, 64, 8, 16385)
    splits = -(-1025 // pps)
    assert n >= 8 * 64 * splits * 132 * 4
    assert kvq.decode_workspace_bytes(8, 64, 8, 16385, 16) >= 8 * 64 * 65 * 132 * 4
    # one split still holds one partial per (sequence, query head)
    assert kvq.decode_workspace_bytes(1, 8, 1, 32, 2) >= 8 * 132 * 4
    with pytest.raises(kvq.KvqError):
        kvq.decode_workspace_bytes(8, 60, 8, 16385)        # Hq % Hkv != 0
    with pytest.raises(kvq.KvqError):
        kvq.decode_workspace_bytes(8, 64, 8, 16385, 3)     # odd split
    with pytest.raises(kvq.KvqError):
        kvq.decode_workspace_bytes(8, 64, 8, 16385, 514)   # above 512 pages per split
    assert kvq.decode_workspace_bytes(1, 8, 1, 1 << 20, 512) > 0
    # the heuristic stays within 512 pages per split even for one long sequence
    assert kvq.decode_pages_per_split(1, 8, 8, 1 << 24) <= 512


def test_split_plan_counts_two_head_groups_per_workgroup():
    """The quantised decode serves two head groups (16 query heads of a KV
    head) per work-group, so the split plan counts work-groups, not head
    groups: 16 heads per KV head plan like 8, and 24 or 32 heads like two
    work-groups (half the splits of one).  The fp16 kernel keeps one group
    per work-group."""
    n = 1 << 16                                  # 4096 pages of one sequence
    p8, p16, p24, p32 = (kvq.decode_pages_per_split(1, h, 1, n) for h in (8, 16, 24, 32))
    assert p16 == p8
    assert p24 == p32
    assert p24 == kvq.decode_pages_per_split(2, 8, 1, n)       # two work-groups per unit
    # slots per row: the same for 8 and 16 quantised heads; the fp16 kernel's
    # two work-groups for 16 heads take half the splits each
    k8, k16 = (kvq.decode_split_slots(1, h, 1, n) for h in (8, 16))
    assert k16 == k8
    f16 = kvq.format_from_string("fp16")
    h8, h16 = (kvq.decode_split_slots(1, h, 1, n, fmt=f16) for h in (8, 16))
    assert h16 < h8


def _fmt():
    return ctypes.byref(kvq.format_from_string())


def test_append_validation_launches_nothing():
    lib = kvq.load()
    P = ctypes.c_void_p
    good = P(0x10000)
    # null format / unsupported format
    assert lib.kvq_quantize_append(None, good, good, 1024, 1024, good, 4, 8, good, 10, None) == 1
    bad = kvq.Format(128, 128, 8, 8, 16)
    assert lib.kvq_quantize_append(ctypes.byref(bad), good, good, 1024, 1024, good, 4, 8, good, 10, None) == 3
    # zero tokens: no-op success
    assert lib.kvq_quantize_append(_fmt(), None, None, 1024, 1024, None, 0, 8, None, 10, None) == 0
    assert lib.kvq_quantize_append(_fmt(), None, good, 1024, 1024, good, 4, 8, good, 10, None) == 1
    assert lib.kvq_quantize_append(_fmt(), good, good, 100, 1024, good, 4, 8, good, 10, None) == 2
    assert lib.kvq_quantize_append(_fmt(), good, good, 1024, 1024, good, -1, 8, good, 10, None) == 2
    assert lib.kvq_quantize_append(_fmt(), P(0x10002), good, 1024, 1024, good, 4, 8, good, 10, None) == 4
    assert lib.kvq_quantize_append(_fmt(), good, good, 1028, 1024, good, 4, 8, good, 10, None) == 2 or \
        lib.kvq_quantize_append(_fmt(), good, good, 1028, 1024, good, 4, 8, good, 10, None) == 4


def test_decode_validation_launches_nothing():
    lib = kvq.load()
    P = ctypes.c_void_p
    g = P(0x10000)
    ws = kvq.decode_workspace_bytes(2, 8, 2, 100)

    def call(**kw):
        a = dict(out=g, dt=1, q=g, cache=g, np=10, bt=g, mp=7, sl=g, B=2, Hq=8, Hkv=2, L=100,
                 scale=0.088, ws=g, wsb=ws, pps=0)
        a.update(kw)
        return lib.kvq_decode_attention_ex(_fmt(), a["out"], a["dt"], a["q"], a["cache"], a["np"], a["bt"],
                                           a["mp"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["L"], a["scale"],
                                           a["ws"], a["wsb"], a["pps"], None)

    assert call(out=None) == 1
    assert call(Hq=7) == 2                      # Hq % Hkv != 0
    assert call(B=0) == 2
    assert call(L=200) == 2                     # max_seq_len > max_pages * 16
    assert call(pps=3) == 2
    assert call(pps=514) == 2
    assert call(dt=5) == 3
    assert call(q=P(0x10008)) == 4
    assert call(wsb=ws - 1) == 5
    assert call(ws=None) == 5
    assert lib.kvq_decode_attention(None, g, 1, g, g, 10, g, 7, g, 2, 8, 2, 100, 0.1, g, ws, None) == 1


def test_two_phase_validation_launches_nothing():
    lib = kvq.load()
    P = ctypes.c_void_p
    g = P(0x10000)
    ws = kvq.decode_workspace_bytes(2, 8, 2, 100)

    def part(**kw):
        a = dict(q=g, cache=g, np=10, bt=g, mp=7, sl=g, B=2, Hq=8, Hkv=2, L=100, scale=0.088,
                 ws=g, wsb=ws, pps=0)
        a.update(kw)
        return lib.kvq_decode_partials(_fmt(), a["q"], a["cache"], a["np"], a["bt"], a["mp"], a["sl"],
                                       a["B"], a["Hq"], a["Hkv"], a["L"], a["scale"], a["ws"], a["wsb"],
                                       a["pps"], None)

    def comb(**kw):
        a = dict(out=g, dt=0, sl=g, B=2, Hq=8, Hkv=2, L=100, ws=g, wsb=ws, pps=0)
        a.update(kw)
        return lib.kvq_decode_combine(_fmt(), a["out"], a["dt"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["L"],
                                      a["ws"], a["wsb"], a["pps"], None)

    assert part(q=None) == 1 and part(bt=None) == 1 and part(sl=None) == 1
    assert part(Hq=6, Hkv=4) == 2 and part(L=200) == 2 and part(mp=0) == 2 and part(np=0) == 2
    assert part(pps=5) == 2 and part(scale=float("nan")) == 2
    assert part(cache=P(0x10004)) == 4 and part(sl=P(0x10002)) == 4
    assert part(wsb=ws - 1) == 5 and part(ws=None) == 5
    assert comb(out=None) == 1 and comb(sl=None) == 1
    assert comb(dt=7) == 3 and comb(B=0) == 2 and comb(pps=1) == 2
    assert comb(out=P(0x10008)) == 4
    assert comb(wsb=16) == 5
    assert lib.kvq_decode_partials(None, g, g, 10, g, 7, g, 2, 8, 2, 100, 0.1, g, ws, 0, None) == 1
    bad = kvq.Format(128, 64, 4, 2, 16)
    assert lib.kvq_decode_combine(ctypes.byref(bad), g, 0, g, 2, 8, 2, 100, g, ws, 0, None) == 3


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the error path of a GPU-less host")
def test_launch_without_gpu_reports_hip_error():
    lib = kvq.load()
    P = ctypes.c_void_p
    g = P(0x10000)
    st = lib.kvq_quantize_append(_fmt(), g, g, 1024, 1024, g, 4, 8, g, 10, None)
    assert st == 6
    assert lib.kvq_last_hip_error() != 0
    assert lib.kvq_status_string(6) == b"HIP runtime error"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    mod = importlib.reload(kvq)
    monkeypatch.setattr(mod, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(RuntimeError):
        mod.load()
    importlib.reload(kvq)


def test_fused_append_validation_launches_nothing():
    lib = kvq.load()
    P = ctypes.c_void_p
    g = P(0x10000)
    ws = kvq.decode_workspace_bytes(2, 8, 2, 100)

    def full(**kw):
        a = dict(out=g, dt=1, k=g, v=g, ks=256, vs=256, q=g, cache=g, np=10, bt=g, mp=7, sl=g, B=2, Hq=8,
                 Hkv=2, L=100, scale=0.088, ws=g, wsb=ws, pps=0)
        a.update(kw)
        return lib.kvq_append_decode_attention(_fmt(), a["out"], a["dt"], a["k"], a["v"], a["ks"], a["vs"],
                                               a["q"], a["cache"], a["np"], a["bt"], a["mp"], a["sl"], a["B"],
                                               a["Hq"], a["Hkv"], a["L"], a["scale"], a["ws"], a["wsb"],
                                               a["pps"], None)

    def part(**kw):
        a = dict(k=g, v=g, ks=256, vs=256, q=g, cache=g, np=10, bt=g, mp=7, sl=g, B=2, Hq=8, Hkv=2, L=100,
                 scale=0.088, ws=g, wsb=ws, pps=0)
        a.update(kw)
        return lib.kvq_append_decode_partials(_fmt(), a["k"], a["v"], a["ks"], a["vs"], a["q"], a["cache"],
                                              a["np"], a["bt"], a["mp"], a["sl"], a["B"], a["Hq"], a["Hkv"],
                                              a["L"], a["scale"], a["ws"], a["wsb"], a["pps"], None)

    for f in (full, part):
        assert f(k=None) == 1 and f(v=None) == 1 and f(q=None) == 1
        assert f(ks=255) == 2 and f(vs=128) == 2           # below num_kv_heads * 128
        assert f(ks=260) == 4                              # not a multiple of 8
        assert f(k=P(0x10008)) == 4
        assert f(cache=P(0x10010)) == 4                    # 16- but not 128-byte aligned
        assert f(Hq=6, Hkv=4) == 2 and f(L=200) == 2
        assert f(wsb=ws - 1) == 5
    assert full(out=None) == 1 and full(dt=9) == 3


def test_fp16_baseline_format():
    lib = kvq.load()
    f = kvq.Format()
    assert lib.kvq_format_from_string(b"fp16", ctypes.byref(f)) == 0
    assert (f.head_dim, f.group_size, f.k_bits, f.v_bits, f.block_size) == (128, 128, 16, 16, 16)
    assert kvq.page_bytes(f) == 8192 == 16 * 128 * 2 * 2
    assert kvq.cache_bytes(10, 8, f) == 10 * 8 * 8192
    # 512 bytes per token per KV head against K4V2's 104
    assert kvq.page_bytes(f) / 16 == 512 and kvq.page_bytes() / 16 == 104
    # splits hold at most 256 fp16 pages
    assert kvq.decode_workspace_bytes(1, 8, 1, 1 << 20, 256, f) > 0
    with pytest.raises(kvq.KvqError):
        kvq.decode_workspace_bytes(1, 8, 1, 1 << 20, 258, f)
    # the fused append-and-decode exists for K4V2 only
    P = ctypes.c_void_p
    g = P(0x10000)
    ws = kvq.decode_workspace_bytes(2, 8, 2, 100, 0, f)
    assert lib.kvq_append_decode_partials(ctypes.byref(f), g, g, 256, 256, g, g, 10, g, 7, g, 2, 8, 2, 100,
                                          0.088, g, ws, 0, None) == 3



def test_multi_query_validation_launches_nothing():
    lib = kvq.load()
    P = ctypes.c_void_p
    g = P(0x10000)
    assert kvq.decode_workspace_bytes_mq(2, 4, 8, 2, 100) == kvq.decode_workspace_bytes(2, 32, 2, 100)
    for bad in ((2, 0, 8, 2, 100), (2, 17, 8, 2, 100), (2, 4, 7, 2, 100)):
        with pytest.raises(kvq.KvqError):
            kvq.decode_workspace_bytes_mq(*bad)
    ws = kvq.decode_workspace_bytes_mq(2, 4, 8, 2, 100)

    def call(fmt=None, **kw):
        a = dict(out=g, dt=1, q=g, M=4, cache=g, np=10, bt=g, mp=7, sl=g, B=2, Hq=8, Hkv=2, L=100,
                 scale=0.088, ws=g, wsb=ws, pps=0)
        a.update(kw)
        f = ctypes.byref(fmt or kvq.format_from_string())
        return lib.kvq_decode_attention_mq(f, a["out"], a["dt"], a["q"], a["M"], a["cache"], a["np"], a["bt"],
                                           a["mp"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["L"], a["scale"],
                                           a["ws"], a["wsb"], a["pps"], None)

    assert call(M=0) == 2 and call(M=17) == 2
    assert call(Hq=7) == 2
    assert call(fmt=kvq.format_from_string("fp16")) == 3      # one query row only for the fp16 baseline
    assert call(out=None) == 1
    assert call(wsb=ws - 1) == 5                              # the workspace of q_len * Hq heads
    assert call(q=P(0x10008)) == 4


@pytest.mark.parametrize("P", [16, 32, 64, 128])
def test_page_sizes(P):
    """Pages of P tokens: P / 16 regions per (page, KV head)."""
    f = kvq.format_from_string("k4v2_g128", page_tokens=P)
    assert f.block_size == P and kvq.page_bytes(f) == P // 16 * 1664
    f84 = kvq.format_from_string("k8v4_g128", page_tokens=P)
    assert kvq.page_bytes(f84) == P // 16 * 3200
    with pytest.raises(kvq.KvqError):
        kvq.format_from_string("fp16", page_tokens=32)
    # max_seq_len may reach max_pages_per_seq * P
    lib = kvq.load()
    g = ctypes.c_void_p(0x10000)
    ws = kvq.decode_workspace_bytes(2, 8, 2, 4 * P, fmt=f)
    st = lib.kvq_decode_attention_ex(ctypes.byref(f), None, 1, g, g, 10, g, 4, g, 2, 8, 2, 4 * P, 0.088, g,
                                     ws, 0, None)
    assert st == 1                      # the sizes pass; the NULL output is reported
    st = lib.kvq_decode_attention_ex(ctypes.byref(f), None, 1, g, g, 10, g, 4, g, 2, 8, 2, 4 * P + 1, 0.088, g,
                                     ws, 0, None)
    assert st == 2                      # 4 pages of P tokens hold at most 4 P


def test_stream_read_probe_validation_launches_nothing():
    lib = kvq.load()
    P = ctypes.c_void_p
    g = P(0x10000)
    assert lib.kvq_stream_read_probe(None, 16, g, None) == 1
    assert lib.kvq_stream_read_probe(g, 16, None, None) == 1
    assert lib.kvq_stream_read_probe(g, 0, g, None) == 2
    assert lib.kvq_stream_read_probe(g, 24, g, None) == 2
    assert lib.kvq_stream_read_probe(g, (1 << 40) + 16, g, None) == 2
    assert lib.kvq_stream_read_probe(P(0x10008), 16, g, None) == 4
    assert lib.kvq_stream_read_probe(g, 16, P(0x10002), None) == 4


def test_page_walk_probe_validation_launches_nothing():
    lib = kvq.load()
    P = ctypes.c_void_p
    g, gs = P(0x10000), P(0x20000)
    f = kvq.format_from_string()
    fb = ctypes.byref(f)

    def call(fmt=fb, cache=g, num_pages=64, bt=g, maxp=40, lens=g, B=2, Hkv=2, max_len=640, pps=8, sink=gs):
        return lib.kvq_page_walk_probe(fmt, cache, num_pages, bt, maxp, lens, B, Hkv, max_len, pps, sink, None)

    assert call(fmt=None) == 1
    assert call(fmt=ctypes.byref(kvq.format_from_string("fp16"))) == 3
    assert call(fmt=ctypes.byref(kvq.format_from_string(page_tokens=32))) == 3
    assert call(cache=None) == 1
    assert call(bt=None) == 1
    assert call(lens=None) == 1
    assert call(sink=None) == 1
    assert call(num_pages=0) == 2
    assert call(B=0) == 2
    assert call(Hkv=0) == 2
    assert call(max_len=0) == 2
    assert call(maxp=0) == 2
    assert call(max_len=641) == 2          # 40 pages of 16 tokens hold at most 640
    for pps in (0, 1, 7, 514):
        assert call(pps=pps) == 2
    assert call(maxp=1 << 24, max_len=(1 << 24) * 16, pps=2) == 2    # more than 65535 splits
    assert call(cache=P(0x10008)) == 4
    assert call(bt=P(0x10002)) == 4
    assert call(lens=P(0x10001)) == 4
    assert call(sink=P(0x20002)) == 4


def test_binding_refuses_host_tensors():
    """The binding never hands a host pointer to a kernel."""
    k = torch.zeros((1, 1, 128), dtype=torch.float16)
    slots = torch.zeros(1, dtype=torch.int64)
    cache = torch.zeros((1, 1, 1664), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensors"):
        kvq.quantize_append(k, k, slots, cache)


def test_noalloc_step_rejects_partials_beyond_its_array_without_a_device():
    """kvq_append_decode_attention_noalloc checks the partials' size against
    its fixed array before it touches the device: sizes whose partials exceed
    KVQ_NOALLOC_SCRATCH_BYTES give KVQ_ERR_WORKSPACE, a NULL format
    KVQ_ERR_NULL, invalid sizes the workspace call's statuses."""
    lib = kvq.load()
    f = kvq.format_from_string("k4v2_g128")
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    g = P(0x10000)

    def call(fmt, B, Hq, Hkv, L, pps=0):
        return lib.kvq_append_decode_attention_noalloc(fmt, g, 1, g, g, i64(Hkv * 128), i64(Hkv * 128), g, g,
                                                       i64(100), g, i32(-(-L // 16)), g, i32(B), i32(Hq), i32(Hkv),
                                                       i32(L), ctypes.c_float(0.088), i32(pps), None)
    assert kvq.decode_workspace_bytes(64, 64, 8, 131072) > kvq.NOALLOC_SCRATCH_BYTES
    assert call(ctypes.byref(f), 64, 64, 8, 131072) == 5
    assert call(None, 8, 64, 8, 1000) == 1
    assert call(ctypes.byref(f), 8, 60, 8, 1000) == 2          # 60 % 8 != 0
    header = open(HEADER).read()
    m = re.search(r"#define KVQ_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", header)
    assert m and int(m.group(1)) << int(m.group(2)) == kvq.NOALLOC_SCRATCH_BYTES


def test_page_balanced_format_and_unsupported_calls_launch_nothing():
    """The page-balanced preset: 1792-byte regions, 16-token pages only, and
    the calls it lacks (fused append-and-decode, several query rows) refused
    before anything is launched."""
    lib = kvq.load()
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    g = P(0x10000)
    for name in ("k4v2_g128_pb", "kvarn_k4v2_g128_pb"):
        f = kvq.format_from_string(name)
        assert (f.k_bits, f.v_bits, f.block_size, f.key_norm) == (4, 2, 16, kvq.KEY_NORM_PAGE)
        assert kvq.page_bytes(f) == 1792 and kvq.cache_bytes(10, 8, f) == 10 * 8 * 1792
    with pytest.raises(kvq.KvqError):
        kvq.format_from_string("k4v2_g128_pb", page_tokens=64)
    f = kvq.format_from_string("k4v2_g128")
    assert f.key_norm == kvq.KEY_NORM_GROUP
    bad = kvq.Format(128, 128, 8, 4, 16, kvq.KEY_NORM_PAGE)      # page-balanced keys are K4V2 only
    assert lib.kvq_page_bytes(ctypes.byref(bad)) == 0
    bad = kvq.Format(128, 128, 4, 2, 16, 2)
    assert lib.kvq_page_bytes(ctypes.byref(bad)) == 0
    pb = ctypes.byref(kvq.format_from_string("k4v2_g128_pb"))
    ws = lib.kvq_decode_workspace_bytes(pb, 2, 8, 2, 100, 0)
    assert ws > 0
    st = lib.kvq_append_decode_attention(pb, g, 1, g, g, i64(256), i64(256), g, g, i64(10), g, i32(7), g, i32(2),
                                         i32(8), i32(2), i32(100), ctypes.c_float(0.088), g, ctypes.c_size_t(ws),
                                         i32(0), None)
    assert st == 3
    st = lib.kvq_append_decode_attention_noalloc(pb, g, 1, g, g, i64(256), i64(256), g, g, i64(10), g, i32(7), g,
                                                 i32(2), i32(8), i32(2), i32(100), ctypes.c_float(0.088), i32(0),
                                                 None)
    assert st == 3
    wsm = lib.kvq_decode_workspace_bytes_mq(pb, 2, 4, 8, 2, 100, 0)
    st = lib.kvq_decode_attention_mq(pb, g, 1, g, i32(4), g, i64(10), g, i32(7), g, i32(2), i32(8), i32(2),
                                     i32(100), ctypes.c_float(0.088), g, ctypes.c_size_t(wsm), i32(0), None)
    assert st == 3
