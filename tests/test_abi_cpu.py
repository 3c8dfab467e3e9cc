"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host before any launch (CPU only: no compute calls)."""
import os
import re

import pytest

import oracle
from long_context_anchor_amd import kascade as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kascade.h")

pytestmark = pytest.mark.skipif(not os.path.exists(K.LIB_PATH), reason="libkascade.so not built")

FAKE = 0x10000  # 16-byte aligned non-null address; validation never dereferences it


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kascade_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = K.lib()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(K.EXPORTS) == names


def test_version_and_status_strings():
    assert K.kascade_version().startswith("kascade")
    assert K.kascade_status_str(0) == "ok"
    assert "workspace" in K.kascade_status_str(-6)


def _shape(B=1, Hq=4, Hkv=2, d=64, N=1024, dtype=K.KASCADE_F32, prefill=False):
    qsn = d if prefill else 0
    qsh = N * d if prefill else d
    return K.Shape(B, Hq, Hkv, d, N, dtype, 0.0, 0, Hq * qsh, qsh, qsn, Hkv * N * d, N * d, d)


def test_topk_rule_matches_oracle():
    r = K.PREFILL_RULE
    for n in (1, 100, 128, 256, 2816, 2944, 32768, 65536, 131072):
        assert K.kascade_topk_for_len(n, r) == oracle.topk_for_len(n, 10, 64, 256)
    dec = K.TopkRule(128, 10, 64, 128)
    for n in (1024, 32768, 131072):
        assert K.kascade_topk_for_len(n, dec) == oracle.topk_for_len(n)
    assert K.kascade_topk_for_len(10, K.TopkRule(128, 0, 64, 256)) == -1


def test_workspace_sizes():
    sh = _shape(N=32768, d=128, Hq=32, Hkv=8, dtype=K.KASCADE_BF16)
    ws = K.kascade_workspace_bytes(K.OP_ANCHOR_DECODE, sh, 3264)
    # at least the spilled scores (B*Hq*N fp32) and the pooled rows (B*Hkv*N fp32)
    assert ws >= 32 * 32768 * 4 + 8 * 32768 * 4
    assert K.kascade_workspace_bytes(K.OP_REUSE_DECODE, sh, 3264) > 0
    assert K.kascade_workspace_bytes(K.OP_ANCHOR_DECODE, _shape(Hq=3), 10) == 0
    sp = _shape(N=4096, d=128, Hq=32, Hkv=8, dtype=K.KASCADE_BF16, prefill=True)
    assert K.kascade_workspace_bytes(K.OP_ANCHOR_PREFILL, sp, 0, K.PREFILL_RULE) >= 32 * 4096 * 4
    assert K.kascade_workspace_bytes(K.OP_ANCHOR_PREFILL, sp, 0, None) == 0


def test_anchor_decode_validation():
    sh = _shape()
    ws_n = K.kascade_workspace_bytes(K.OP_ANCHOR_DECODE, sh, 128)
    call = lambda **kw: K.kascade_anchor_decode(
        kw.get("shape", sh), kw.get("q", FAKE), FAKE, FAKE, kw.get("topk", 128), FAKE, None,
        kw.get("idx", FAKE), None, FAKE, kw.get("ws", ws_n), 0)
    assert call(q=None) == -1
    assert call(idx=None) == -1
    assert call(topk=0) == -4
    assert call(topk=1025) == -4
    assert call(ws=ws_n - 1) == -6
    assert call(shape=_shape(Hq=3)) == -2
    assert call(shape=_shape(Hq=12, Hkv=4)) == -2      # group of 3 unsupported
    assert call(shape=_shape(d=128)) == -3             # fp32 needs d = 64
    assert call(shape=_shape(d=64, dtype=K.KASCADE_BF16)) == -3
    assert call(q=FAKE + 8) == -8                       # misaligned pointer
    bad = _shape()
    bad.kv_stride_n = 60
    assert call(shape=bad) == -2


def test_anchor_decode_fused_validation():
    """The one-launch anchor decode rejects bad arguments before any device call."""
    sh = _shape(N=4096, d=128, Hq=8, Hkv=2, dtype=K.KASCADE_BF16)
    ws_n = K.kascade_workspace_bytes(K.OP_ANCHOR_DECODE_FUSED, sh, 128)
    # status word, counters, partials for 256 splits, two histograms, candidates, counts
    assert ws_n >= 256 + 256 * 64 * 4 + 8 * 256 * 130 * 4 + 2 * 2 * 2048 * 4 + 2 * 4096 * 4
    call = lambda **kw: K.kascade_anchor_decode_fused(
        kw.get("shape", sh), kw.get("q", FAKE), FAKE, FAKE, kw.get("topk", 128), FAKE, None,
        kw.get("idx", FAKE), None, 0, FAKE, kw.get("ws", ws_n), 0)
    assert call(q=None) == -1
    assert call(idx=None) == -1
    assert call(topk=0) == -4
    assert call(topk=4097) == -4
    assert call(ws=ws_n - 1) == -6
    assert call(shape=_shape(N=4096, d=64, Hq=8, Hkv=2)) == -3      # fp32 caches: not fused
    assert call(shape=_shape(N=4096, d=128, Hq=12, Hkv=4, dtype=K.KASCADE_BF16)) == -2
    assert call(q=FAKE + 8) == -8


def test_reuse_decode_validation():
    sh = _shape()
    ws_n = K.kascade_workspace_bytes(K.OP_REUSE_DECODE, sh, 128)
    call = lambda hm, topk=128, ws=ws_n: K.kascade_reuse_decode(sh, FAKE, FAKE, FAKE, topk, FAKE, hm,
                                                              FAKE, FAKE, ws, 0)
    assert call([0, 2]) == -5
    assert call([-1, 0]) == -5
    assert call(None) == -1
    assert call([0, 1], topk=2000) == -4
    assert call([0, 1], ws=0) == -6


def test_prefill_validation():
    sp = _shape(N=1000, d=128, Hq=8, Hkv=2, dtype=K.KASCADE_BF16, prefill=True)
    ws_n = K.kascade_workspace_bytes(K.OP_ANCHOR_PREFILL, sp, 0, K.PREFILL_RULE)
    call = lambda rule=K.PREFILL_RULE, shape=sp, ws=ws_n: K.kascade_anchor_prefill(
        shape, FAKE, FAKE, FAKE, rule, FAKE, None, FAKE, None, FAKE, ws, 0)
    assert call(rule=K.TopkRule(64, 10, 64, 256)) == -4     # tile must be 128
    assert call(rule=K.TopkRule(128, 10, 64, 64)) == -4     # k_min below the tile
    assert call(ws=ws_n - 1) == -6
    assert call(shape=_shape(N=1000, d=64, prefill=True)) == -3  # fp32 prefill unsupported
    wide = _shape(N=64, d=128, Hq=8, Hkv=2, dtype=K.KASCADE_BF16, prefill=True)
    wide.kv_stride_n = (1 << 24) + 8       # rows of 32 MiB + 16 B: a 64-row block spans 2 GiB
    wide.kv_stride_h = wide.kv_stride_n * 64
    wide.kv_stride_b = wide.kv_stride_h * 2
    assert call(shape=wide) == -2
    wide.kv_stride_n = 1 << 24              # exactly 32 MiB rows pass the shape check: the call
    wide.kv_stride_h = wide.kv_stride_n * 64  # then stops at the (short) workspace, before any launch
    wide.kv_stride_b = wide.kv_stride_h * 2
    need = K.kascade_workspace_bytes(K.OP_ANCHOR_PREFILL, wide, 0, K.PREFILL_RULE)
    assert need > 0 and call(shape=wide, ws=need - 1) == -6
    assert K.kascade_reuse_prefill(sp, FAKE, FAKE, FAKE, K.PREFILL_RULE, FAKE, [0, 5], FAKE,
                                   None, 0, 0) == -5


def test_select_validation():
    assert K.kascade_topk_select_f32(FAKE, 10, 4, 10, 0, FAKE, 10, 0) == -4
    assert K.kascade_topk_select_f32(FAKE, 10, 4, 10, 11, FAKE, 11, 0) == -4
    assert K.kascade_topk_select_f32(FAKE, 5, 4, 10, 3, FAKE, 3, 0) == -2
    assert K.kascade_topk_select_f32(None, 10, 4, 10, 3, FAKE, 3, 0) == -1
    assert K.kascade_topk_select_f32(FAKE, 10, 0, 10, 3, FAKE, 3, 0) == 0   # nothing to do


def test_stream_read_validation():
    assert K.kascade_stream_read(None, 64, FAKE, 0) == -1
    assert K.kascade_stream_read(FAKE, 64, None, 0) == -1
    assert K.kascade_stream_read(FAKE, 0, FAKE, 0) == -8          # empty
    assert K.kascade_stream_read(FAKE, 24, FAKE, 0) == -8         # not whole 16-byte words
    assert K.kascade_stream_read(FAKE + 8, 64, FAKE, 0) == -8     # source not 16-byte aligned
    assert K.kascade_stream_read(FAKE, 64, FAKE + 2, 0) == -8     # sink not 4-byte aligned


def test_timer_api_bounds():
    assert K.lib().kascade_kernel_timer_enable(99, 1) == -8


def test_paged_decode_validation_errors():
    """Paged entry points reject bad descriptors before any device call."""
    sh = _shape(N=1000, d=128, Hq=8, Hkv=2, dtype=K.KASCADE_BF16)
    sh.kv_stride_b = 0
    sh.kv_stride_h = 16 * 128
    ws = 1 << 30

    def desc(**kw):
        pg = K.PagedKV(FAKE, 70, 16, 200, 0, 2 * 16 * 128)
        for f, v in kw.items():
            setattr(pg, f, v)
        return pg

    def anchor(pg, shape=sh):
        return K.kascade_anchor_decode_paged(shape, pg, FAKE, FAKE, FAKE, 10, FAKE, None, FAKE, None, FAKE,
                                             ws, 0)

    assert anchor(desc(block_size=24)) == -2        # not a power of two
    assert anchor(desc(table_stride=10)) == -2      # table shorter than ceil(N / block_size)
    assert anchor(desc(reserved=1)) == -8
    assert anchor(desc(block_stride=100)) == -2     # not a multiple of the row stride
    assert anchor(desc(block_stride=16 * 128)) == -2    # second head's rows outside the block
    assert anchor(desc(block_table=None)) == -1
    assert anchor(desc(block_size=32), shape=_shape(N=1000)) == -3   # fp32 caches are not paged
    assert K.kascade_reuse_decode_paged(sh, desc(block_table=None), FAKE, FAKE, FAKE, 10, FAKE, [0, 1], FAKE,
                                        FAKE, ws, 0) == -1


def test_paged_reuse_prefill_validation_errors():
    """The paged reuse prefill checks the descriptor, rule, head map and list
    length on the host; every call below stops before a launch."""
    sp = _shape(N=1000, d=128, Hq=8, Hkv=2, dtype=K.KASCADE_BF16, prefill=True)
    sp.kv_stride_b = 0
    sp.kv_stride_h = 16 * 128

    def desc(**kw):
        pg = K.PagedKV(FAKE, 70, 16, 200, 0, 2 * 16 * 128)
        for f, v in kw.items():
            setattr(pg, f, v)
        return pg

    def call(pg, shape=sp, rule=K.PREFILL_RULE, hm=(0, 1)):
        return K.kascade_reuse_prefill_paged(shape, pg, FAKE, FAKE, FAKE, rule, FAKE, list(hm), FAKE, None, 0, 0)

    assert K.lib().kascade_reuse_prefill_paged(None, None, None, None, None, None, None, None, None,
                                               None, 0, None) == -1
    assert call(desc(block_table=None)) == -1
    assert call(desc(block_size=24)) == -2            # not a power of two
    assert call(desc(table_stride=10)) == -2          # table shorter than ceil(N / block_size)
    assert call(desc(block_stride=16 * 128)) == -2    # second head's rows outside the block
    assert call(desc(reserved=1)) == -8
    assert call(desc(), rule=K.TopkRule(128, 10, 64, 64)) == -4
    assert call(desc(), hm=(0, 2)) == -5
    # k of the last tile above the paged list bound (12288 keys): 10% of 130000 tokens
    long = _shape(N=130000, d=128, Hq=8, Hkv=2, dtype=K.KASCADE_BF16, prefill=True)
    long.kv_stride_b = 0
    long.kv_stride_h = 16 * 128
    assert K.kascade_topk_for_len(130000, K.PREFILL_RULE) > 12288
    assert call(desc(table_stride=-(-130000 // 16), num_blocks=20000), shape=long) == -2
