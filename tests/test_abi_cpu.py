"""The C ABI library loads, exports every declared symbol, and rejects bad calls
on the host before touching a device (CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

from mqa_decode_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

KVC_OK, KVC_ERR_NULL, KVC_ERR_SHAPE, KVC_ERR_UNSUPPORTED, KVC_ERR_WORKSPACE, KVC_ERR_HIP = range(6)
F32, BF16, U8 = 0, 1, 2
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails its host checks


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must mirror the header"


def test_version_and_status_strings(lib):
    assert lib.kvc_abi_version() == _lib.ABI_VERSION == 14
    for s in range(6):
        assert lib.kvc_status_string(s)
    assert lib.kvc_status_string(99) == b"unknown status"
    assert lib.kvc_last_error() is not None


def _append(lib, **kw):
    a = dict(dt=BF16, B=2, H_q=8, H_kv=2, d=128, k=FAKE, v=FAKE, T_max=64, tbl=None, bs=0, mb=0, nb=0,
             pos=FAKE, kn=FAKE, vn=FAKE, q=None, cos=FAKE, sin=FAKE, rows=64, style=0, stream=None)
    a.update(kw)
    return lib.kvc_append(a["dt"], a["B"], a["H_q"], a["H_kv"], a["d"], a["k"], a["v"], a["T_max"],
                          a["tbl"], a["bs"], a["mb"], a["nb"], a["pos"], a["kn"], a["vn"], a["q"],
                          a["cos"], a["sin"], a["rows"], a["style"], a["stream"])


def test_append_host_checks(lib):
    assert _append(lib, H_q=6, H_kv=4) == KVC_ERR_SHAPE
    assert b"multiple" in lib.kvc_last_error()
    assert _append(lib, d=127) == KVC_ERR_SHAPE
    assert _append(lib, style=7) == KVC_ERR_UNSUPPORTED
    assert _append(lib, dt=5) == KVC_ERR_UNSUPPORTED
    assert _append(lib, k=None) == KVC_ERR_NULL
    assert _append(lib, pos=None) == KVC_ERR_NULL
    assert _append(lib, cos=None) == KVC_ERR_NULL
    assert _append(lib, T_max=0) == KVC_ERR_SHAPE
    assert _append(lib, tbl=FAKE, bs=0, mb=4, nb=10) == KVC_ERR_SHAPE
    assert _append(lib, rows=0) == KVC_ERR_SHAPE
    assert _append(lib, B=0) == KVC_OK           # nothing to do, nothing launched


def _decode(lib, **kw):
    a = dict(dt=BF16, B=2, H_q=8, H_kv=2, d=128, q=FAKE, k=FAKE, v=FAKE, T_max=64, lens=FAKE, L=64,
             scale=0.0, out=FAKE, split=0, ws=None, wsn=0, stream=None)
    a.update(kw)
    return lib.kvc_decode_attn(a["dt"], a["B"], a["H_q"], a["H_kv"], a["d"], a["q"], a["k"], a["v"],
                               a["T_max"], a["lens"], a["L"], a["scale"], a["out"], a["split"], a["ws"],
                               a["wsn"], a["stream"])


def test_decode_host_checks(lib):
    assert _decode(lib, H_q=7) == KVC_ERR_SHAPE
    assert _decode(lib, L=65) == KVC_ERR_SHAPE                  # beyond T_max
    assert b"T_max" in lib.kvc_last_error()
    assert _decode(lib, L=-1) == KVC_ERR_SHAPE
    assert _decode(lib, q=None) == KVC_ERR_NULL
    assert _decode(lib, out=None) == KVC_ERR_NULL
    assert _decode(lib, lens=None) == KVC_ERR_NULL
    assert _decode(lib, d=96) == KVC_ERR_UNSUPPORTED
    assert _decode(lib, d=2) == KVC_ERR_UNSUPPORTED
    assert _decode(lib, dt=9) == KVC_ERR_UNSUPPORTED
    # a long sequence needs splits and therefore a workspace
    assert _decode(lib, T_max=100000, L=100000) == KVC_ERR_WORKSPACE
    need = lib.kvc_decode_workspace_bytes(BF16, 2, 8, 2, 128, 100000, 0, 0)
    assert need > 0
    assert _decode(lib, T_max=100000, L=100000, ws=FAKE, wsn=need - 1) == KVC_ERR_WORKSPACE
    assert _decode(lib, T_max=100000, L=100000, ws=ctypes.c_void_p(0x1008), wsn=need) == KVC_ERR_WORKSPACE
    assert b"aligned" in lib.kvc_last_error()
    # too many splits for the merge step
    assert _decode(lib, T_max=100000, L=100000, split=16) == KVC_ERR_UNSUPPORTED
    assert _decode(lib, B=0) == KVC_OK


def test_paged_host_checks(lib):
    f = lib.kvc_decode_attn_paged
    args = [BF16, 2, 8, 2, 128, FAKE, FAKE, FAKE, 100, 16, FAKE, 4, FAKE, 64, 0.0, FAKE, 0, None, 0, None]
    bad = list(args)
    bad[10] = None
    assert f(*bad) == KVC_ERR_NULL                                # no block table
    bad = list(args)
    bad[13] = 65                                                  # 4 blocks * 16 tokens = 64
    assert f(*bad) == KVC_ERR_SHAPE
    bad = list(args)
    bad[9] = 0
    assert f(*bad) == KVC_ERR_SHAPE


def _window(lib, **kw):
    a = dict(dt=BF16, B=2, H_q=8, H_kv=2, d=128, q=FAKE, k=FAKE, v=FAKE, T_max=64, tbl=None, bs=0, mb=0, nb=0,
             lens=FAKE, L=64, window=16, ring=0, scale=0.0, out=FAKE, split=0, ws=None, wsn=0, stream=None)
    a.update(kw)
    return lib.kvc_decode_attn_window(a["dt"], a["B"], a["H_q"], a["H_kv"], a["d"], a["q"], a["k"], a["v"],
                                      a["T_max"], a["tbl"], a["bs"], a["mb"], a["nb"], a["lens"], a["L"],
                                      a["window"], a["ring"], a["scale"], a["out"], a["split"], a["ws"], a["wsn"],
                                      a["stream"])


def test_window_host_checks(lib):
    """Sliding-window calls: a negative window, a ring with a block table or a
    window other than its T_max slots, a full cache shorter than max_seq_len,
    and the token span that sizes the workspace."""
    span = lib.kvc_window_span
    assert span(5000, 4096, 0, 0) == 4096 + 15
    assert span(100, 4096, 0, 0) == 100
    assert span(5000, 0, 0, 0) == 5000
    assert span(5000, 0, 1, 4096) == 4096
    assert span(100, 4096, 1, 4096) == 100
    assert span(-1, 16, 0, 0) == -1 and span(10, -1, 0, 0) == -1 and span(10, 0, 1, 0) == -1
    assert _window(lib, window=-1) == KVC_ERR_SHAPE
    assert _window(lib, ring=1, tbl=FAKE, bs=16, mb=4, nb=8) == KVC_ERR_UNSUPPORTED
    assert _window(lib, ring=1, window=16) == KVC_ERR_SHAPE            # a ring of 64 slots
    assert b"T_max" in lib.kvc_last_error()
    assert _window(lib, L=65) == KVC_ERR_SHAPE                         # a full cache holds max_seq_len
    assert _window(lib, q=None) == KVC_ERR_NULL
    assert _window(lib, ring=1, window=64, L=100000, q=None) == KVC_ERR_NULL   # a ring takes any length
    # the splits of a window cover its span, not the whole sequence
    assert _window(lib, T_max=100000, L=100000, window=512, B=0) == KVC_OK
    wsb = lib.kvc_decode_workspace_bytes
    assert 0 < wsb(BF16, 2, 8, 2, 128, span(100000, 512, 0, 0), 0, 0) < wsb(BF16, 2, 8, 2, 128, 100000, 0, 0)
    assert _window(lib, dt=U8) == KVC_ERR_UNSUPPORTED or _window(lib, dt=U8) == KVC_ERR_NULL
    ar = lib.kvc_append_ring
    args = [BF16, 2, 8, 2, 128, FAKE, FAKE, 64, FAKE, FAKE, FAKE, None, FAKE, FAKE, 64, 0, None]
    bad = list(args)
    bad[7] = 0
    assert ar(*bad) == KVC_ERR_SHAPE                                   # T_max
    bad = list(args)
    bad[5] = None
    assert ar(*bad) == KVC_ERR_NULL
    bad = list(args)
    bad[1] = 0
    assert ar(*bad) == KVC_OK


def test_workspace_sizes(lib):
    ws = lib.kvc_decode_workspace_bytes
    assert ws(F32, 1, 4, 4, 16, 6, 0, 0) == 0                     # one split, no workspace
    assert ws(BF16, 16, 32, 8, 128, 8193, 0, 0) > 0
    # explicit split: the arrival counters (one per sequence and KV head, in a
    # fixed 64 KiB prefix), then partials for B*H_q heads, n_splits each,
    # d + 2 floats, 256-aligned regions
    zb = lib.kvc_workspace_zeroed_bytes()
    assert zb == 16384 * 4
    n = ws(BF16, 16, 32, 8, 128, 8193, 0, 1024)
    splits = -(-8193 // 1024)
    assert n >= zb + 16 * 32 * splits * (128 + 2) * 4 and n % 256 == 0
    assert n < zb + 16 * 32 * splits * (128 + 2) * 4 + 1024
    assert ws(BF16, 16, 32, 8, 128, 8193, 0, 8193) == 0
    assert ws(BF16, 16, 30, 8, 128, 8193, 0, 0) == (1 << 64) - 1  # invalid sizes
    assert ws(BF16, 16, 32, 8, 128, 8193, -1, 0) == (1 << 64) - 1
    assert ws(BF16, 1, 64, 8, 128, 131073, 0, 0) > 0


def test_split_choice(lib):
    """The library's split length: one balanced round of workgroups (about three
    per slot for groups of more than 16 heads), a floor of 32 * G tokens (12 * G
    for those groups), shorter splits for ragged paged pools, whole loop steps
    of the kernel (64 tokens up to d = 128, else 128).  (The device count is
    256 compute units when no GPU can be queried, as here.)"""
    st = lib.kvc_decode_split_tokens
    # contiguous d = 128: one workgroup per CU, 256 slots
    # (splits are whole 64-token steps)
    # (the last split of a contiguous cache also takes a remainder shorter
    # than one step, so 8193 tokens are 4096 + 4097, not 4160 + 4033)
    wsb = lib.kvc_decode_workspace_bytes
    zb = lib.kvc_workspace_zeroed_bytes()
    assert st(BF16, 16, 32, 8, 128, 8193, 0, 0) == 4096         # 128 units: 2 splits
    assert wsb(BF16, 16, 32, 8, 128, 8193, 0, 0) == zb + 16 * 32 * 2 * (8 + 128 * 4)
    assert st(BF16, 1, 64, 8, 128, 131073, 0, 0) == 4096        # 8 units: 32 splits
    assert wsb(BF16, 1, 64, 8, 128, 131073, 0, 0) == zb + 64 * 32 * (8 + 128 * 4)
    assert st(BF16, 64, 32, 1, 128, 4097, 0, 0) == 384          # G = 32: ~3 per slot, >= 12 * G tokens
    assert st(BF16, 16, 32, 8, 64, 8193, 0, 0) == 2048          # d = 64: two per CU, 512 slots
    assert st(BF16, 16, 32, 8, 256, 8193, 0, 0) == 4096         # d = 256: 128-token steps, 4096 + 4097
    # a remainder of a whole step or more is a split of its own
    assert wsb(BF16, 16, 32, 8, 128, 8193 + 63, 0, 0) == wsb(BF16, 16, 32, 8, 128, 8193, 0, 0)
    assert st(BF16, 16, 32, 8, 128, 8193 + 64, 0, 0) == 4160
    # explicit splits and paged pools keep whole splits: no remainder joins
    assert wsb(BF16, 16, 32, 8, 128, 8193, 0, 4096) == zb + 16 * 32 * 3 * (8 + 128 * 4)
    # one round of workgroups merges in the streaming kernel; more rounds, or
    # the vector kernel, launch a merge kernel; one split needs none
    ml = lib.kvc_decode_merge_launch
    assert ml(BF16, 16, 32, 8, 128, 8193, 0, 0) == 0            # 256 workgroups on 256 slots
    assert ml(BF16, 1, 64, 8, 128, 131073, 0, 0) == 0
    assert ml(U8, 16, 32, 8, 128, 8193, 0, 0) == 0              # 512 on 512
    assert ml(BF16, 64, 32, 1, 128, 4097, 0, 0) == 1            # G = 32: ~3 per slot
    assert ml(BF16, 16, 32, 8, 128, 8193, 0, 1024) == 1         # 1152 workgroups
    assert ml(F32, 16, 32, 8, 128, 8193, 0, 0) == 1             # the vector kernel
    assert ml(BF16, 16, 32, 8, 128, 100, 0, 0) == 0             # one split
    assert ml(BF16, 16, 30, 8, 128, 100, 0, 0) == -1
    assert st(BF16, 16, 32, 8, 128, 8193, 0, 1000) == 1000      # explicit split kept
    # paged pool holding about half of B * max_seq_len tokens: ~4 rounds of
    # splits over 768 slots (three per CU): 17408 * 16 * 8 / (4 * 768) = 725.3 -> 768
    pool = 17408 * 16
    assert st(BF16, 32, 32, 8, 128, 16385, pool, 0) == 768
    # a pool as large as B * max_seq_len gets one round: 256 units on 768 slots, 3 splits
    assert st(BF16, 32, 32, 8, 128, 16385, 32 * 16385, 0) == 5504
    for args in [(BF16, 16, 32, 8, 128, 8193), (BF16, 3, 12, 4, 64, 700), (BF16, 2, 24, 1, 256, 500)]:
        t = st(*args, 0, 0)
        step = 64 if args[4] <= 128 else 128
        G = args[2] // args[3]
        assert t > 0 and t % step == 0 and t >= (12 if G > 16 else 32) * G
    assert st(BF16, 16, 30, 8, 128, 8193, 0, 0) == -1

def test_quantized_cache_host_checks(lib):
    """The uint8-cache entry points check on the host: missing pair arrays, head
    dims without a kernel, paged block sizes that are not a multiple of 16,
    splits spanning more blocks than the staged table slice, sizes."""
    dec = lib.kvc_decode_attn_u8
    #       B  H_q H_kv d    q     kc    ks    vc    vs    T   lens  L   scale out  split ws wsn stream
    args = [2, 8, 2, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 64, 0.0, FAKE, 0, None, 0, None]
    bad = list(args)
    bad[6] = None
    assert dec(*bad) == KVC_ERR_NULL                                  # no K pairs
    bad = list(args)
    bad[8] = None
    assert dec(*bad) == KVC_ERR_NULL                                  # no V pairs
    bad = list(args)
    bad[3] = 256
    assert dec(*bad) == KVC_ERR_UNSUPPORTED                           # head_dim 256: no quantized kernel
    bad = list(args)
    bad[1] = 7
    assert dec(*bad) == KVC_ERR_SHAPE
    bad = list(args)
    bad[11] = 65
    assert dec(*bad) == KVC_ERR_SHAPE                                 # beyond T_max
    bad = list(args)
    bad[0] = 0
    assert dec(*bad) == KVC_OK
    pg = lib.kvc_decode_attn_paged_u8
    #        B  H_q H_kv d    q     kc    ks    vc    vs    nblk bs  tbl  mb lens  L   scale out  split ws  wsn stream
    pargs = [2, 8, 2, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 16, FAKE, 4, FAKE, 64, 0.0, FAKE, 0, None, 0, None]
    bad = list(pargs)
    bad[10] = 8
    assert pg(*bad) == KVC_ERR_UNSUPPORTED                            # block size 8
    bad = list(pargs)
    bad[11] = None
    assert pg(*bad) == KVC_ERR_NULL
    bad = list(pargs)
    bad[17] = 40
    assert pg(*bad) == KVC_ERR_UNSUPPORTED                            # split of 40 tokens
    big = list(pargs)
    big[12], big[14], big[17] = 2000, 32000, 1 << 20                 # a split over 2000 blocks
    assert pg(*big) == KVC_ERR_UNSUPPORTED
    app = lib.kvc_append_u8
    #        dt   B  H_q H_kv d    kc    ks    vc    vs    T   tbl  bs mb nblk pos   kn    vn    q     cos   sin   rows style stream
    aargs = [BF16, 2, 8, 2, 128, FAKE, FAKE, FAKE, FAKE, 64, None, 0, 0, 0, FAKE, FAKE, FAKE, None, FAKE, FAKE, 64, 0, None]
    bad = list(aargs)
    bad[6] = None
    assert app(*bad) == KVC_ERR_NULL
    bad = list(aargs)
    bad[4] = 258
    assert app(*bad) == KVC_ERR_SHAPE                                 # more than 256 elements
    bad = list(aargs)
    bad[1] = 0
    assert app(*bad) == KVC_OK


def test_fp8_cache_host_checks(lib):
    """The FP8 entry points take the uint8 calls' arguments after a format,
    which must be KVC_FP8_E4M3 or KVC_FP8_E5M2; the uint8 rules apply."""
    E4M3, E5M2 = 3, 4
    dec = lib.kvc_decode_attn_fp8
    args = [E4M3, 2, 8, 2, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, 64, 0.0, FAKE, 0, None, 0, None]
    for fmt in (BF16, U8, 0, 5, -1):
        bad = list(args)
        bad[0] = fmt
        assert dec(*bad) == KVC_ERR_UNSUPPORTED                       # not an FP8 format
    bad = list(args)
    bad[7] = None
    assert dec(*bad) == KVC_ERR_NULL                                  # no K pairs
    bad = list(args)
    bad[4] = 256
    assert dec(*bad) == KVC_ERR_UNSUPPORTED                           # head_dim 256: no 8-bit kernel
    for fmt in (E4M3, E5M2):
        ok = list(args)
        ok[0], ok[1] = fmt, 0
        assert dec(*ok) == KVC_OK                                     # nothing to do
    pg = lib.kvc_decode_attn_paged_fp8
    pargs = [E5M2, 2, 8, 2, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 16, FAKE, 4, FAKE, 64, 0.0, FAKE, 0, None, 0,
             None]
    bad = list(pargs)
    bad[11] = 8
    assert pg(*bad) == KVC_ERR_UNSUPPORTED                            # block size 8
    bad = list(pargs)
    bad[0] = BF16
    assert pg(*bad) == KVC_ERR_UNSUPPORTED
    app = lib.kvc_append_fp8
    aargs = [E4M3, BF16, 2, 8, 2, 128, FAKE, FAKE, FAKE, FAKE, 64, None, 0, 0, 0, FAKE, FAKE, FAKE, None, FAKE, FAKE,
             64, 0, None]
    bad = list(aargs)
    bad[0] = U8
    assert app(*bad) == KVC_ERR_UNSUPPORTED
    bad = list(aargs)
    bad[7] = None
    assert app(*bad) == KVC_ERR_NULL
    step = lib.kvc_decode_step_fp8
    sargs = [E4M3, 2, 8, 2, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, None, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
             64, 0, 64, 0.0, FAKE, 0, None, 0, None]
    bad = list(sargs)
    bad[0] = 7
    assert step(*bad) == KVC_ERR_UNSUPPORTED
    # the same plan as the uint8 cache (the same kernel)
    for fmt in (E4M3, E5M2):
        assert lib.kvc_decode_split_tokens(fmt, 16, 32, 8, 128, 8193, 0, 0) == \
            lib.kvc_decode_split_tokens(U8, 16, 32, 8, 128, 8193, 0, 0)
        assert lib.kvc_decode_workspace_bytes(fmt, 64, 32, 1, 128, 4097, 0, 0) == \
            lib.kvc_decode_workspace_bytes(U8, 64, 32, 1, 128, 4097, 0, 0)


def test_quantized_cache_split_choice(lib):
    """The quantized kernel's plan: 128-token steps, two workgroups per CU (one
    for groups of more than 16 heads), the same floors and ragged-pool rule."""
    st = lib.kvc_decode_split_tokens
    assert st(U8, 16, 32, 8, 128, 8193, 0, 0) == 2176                # 512 slots over 128 units: 4 splits
    assert st(U8, 64, 32, 1, 128, 4097, 0, 0) == 384                 # G = 32
    assert st(U8, 32, 32, 8, 128, 16385, 17408 * 16, 0) == 1152      # ragged pool: ~4 rounds
    assert st(U8, 16, 32, 8, 256, 8193, 0, 0) == -1                  # no quantized kernel at d = 256
    assert lib.kvc_decode_workspace_bytes(U8, 16, 32, 8, 128, 8193, 0, 0) > 0


def _mla(lib, **kw):
    a = dict(B=2, H=32, dk=128, dl=512, rd=64, q=FAKE, cache=FAKE, T_max=64, lens=FAKE, max_len=64, wk=FAKE,
             wv=FAKE, bv=None, scale=0.0, out=FAKE, split=0, ws=FAKE, wsn=1 << 30, stream=None)
    a.update(kw)
    return lib.kvc_decode_attn_mla(a["B"], a["H"], a["dk"], a["dl"], a["rd"], a["q"], a["cache"], a["T_max"],
                                   a["lens"], a["max_len"], a["wk"], a["wv"], a["bv"], a["scale"], a["out"],
                                   a["split"], a["ws"], a["wsn"], a["stream"])


def test_latent_cache_host_checks(lib):
    """The latent-cache entry points check sizes, pointers and the workspace on
    the host (every call here fails before a launch)."""
    assert _mla(lib, dl=384) == KVC_ERR_UNSUPPORTED                # no kernel for this latent width
    assert b"d_latent" in lib.kvc_last_error()
    assert _mla(lib, dk=48) == KVC_ERR_UNSUPPORTED                 # d_k not a multiple of 32
    assert _mla(lib, rd=3) == KVC_ERR_SHAPE                        # rows not 16-byte multiples
    assert _mla(lib, max_len=65) == KVC_ERR_SHAPE                  # beyond T_max
    assert _mla(lib, split=40) == KVC_ERR_UNSUPPORTED              # split not a multiple of 32
    assert _mla(lib, q=None) == KVC_ERR_NULL
    assert _mla(lib, lens=None) == KVC_ERR_NULL
    assert _mla(lib, ws=None) == KVC_ERR_WORKSPACE
    assert _mla(lib, wsn=1024) == KVC_ERR_WORKSPACE
    assert _mla(lib, ws=ctypes.c_void_p(0x1010)) == KVC_ERR_WORKSPACE   # not 256-byte aligned
    assert _mla(lib, B=0) == KVC_OK                                # nothing to do
    st = lib.kvc_decode_step_mla
    assert st(2, 32, 128, 512, 64, FAKE, FAKE, 64, FAKE, None, FAKE, 64, FAKE, FAKE, None, 0.0, FAKE, 0, FAKE,
              1 << 30, None) == KVC_ERR_NULL                        # no new latent rows
    app = lib.kvc_append_mla
    assert app(BF16, 2, 512, 60, FAKE, 64, FAKE, FAKE, FAKE, None) == KVC_ERR_SHAPE
    assert app(BF16, 2, 512, 64, FAKE, 64, FAKE, FAKE, None, None) == KVC_ERR_NULL
    assert app(U8, 2, 512, 64, FAKE, 64, FAKE, FAKE, FAKE, None) == KVC_ERR_UNSUPPORTED


def test_latent_cache_plan(lib):
    """Splits of the latent-cache decode: about one workgroup per compute unit
    over the sequences and 32-head chunks, at least 256 tokens, whole 32-token
    tiles; the workspace holds the absorbed queries, the merged context and
    the partials."""
    st, ws = lib.kvc_decode_mla_split_tokens, lib.kvc_decode_mla_workspace_bytes
    assert st(16, 32, 512, 8193, 0) == 544                         # 16 sequences: 16 splits each
    assert st(1, 32, 512, 131073, 0) == 544                        # 241 splits (513 -> whole tiles)
    assert st(64, 32, 512, 4097, 0) == 1056                       # 4 splits (1025 -> whole tiles)
    assert st(2, 64, 512, 300, 0) == 256                           # floor of 256 tokens
    assert st(16, 32, 512, 8193, 96) == 96
    rows = 16 * 32
    splits = -(-8193 // 544)
    zb = lib.kvc_workspace_zeroed_bytes()                         # (left to the other decode calls)
    n = ws(16, 32, 512, 8193, 0)
    assert n >= zb + 2 * rows * 512 * 4 + rows * splits * (512 + 2) * 4 and n % 256 == 0
    one = ws(16, 32, 512, 200, 0)                                  # one split: one partial per head
    assert zb + 2 * rows * 512 * 4 + rows * (512 + 2) * 4 <= one < zb + 2 * rows * 512 * 4 + rows * (512 + 2) * 4 + 1024
    assert ws(16, 32, 384, 8193, 0) == (1 << 64) - 1


def _noalloc(lib, **kw):
    a = dict(dt=BF16, B=2, H_q=8, H_kv=2, d=128, q=FAKE, qr=FAKE, k=FAKE, v=FAKE, T_max=4096, tbl=None, bs=0,
             mb=0, nb=0, pos=FAKE, kn=FAKE, vn=FAKE, cos=FAKE, sin=FAKE, rows=4096, style=0, max_len=4096,
             scale=0.0, out=FAKE, split=0, stream=None)
    a.update(kw)
    return lib.kvc_decode_step_noalloc(a["dt"], a["B"], a["H_q"], a["H_kv"], a["d"], a["q"], a["qr"], a["k"],
                                       a["v"], a["T_max"], a["tbl"], a["bs"], a["mb"], a["nb"], a["pos"], a["kn"],
                                       a["vn"], a["cos"], a["sin"], a["rows"], a["style"], a["max_len"],
                                       a["scale"], a["out"], a["split"], a["stream"])


def test_noalloc_step_host_checks(lib):
    """The entry point that allocates nothing refuses, on the host, a call whose
    split partials would not fit its fixed array, and names invalid sizes as
    kvc_decode_step does."""
    cap = lib.kvc_decode_step_noalloc_max_bytes()
    assert cap == 32 << 20
    need = lib.kvc_decode_workspace_bytes(BF16, 64, 64, 8, 128, 4096, 0, 16)
    assert need > cap
    assert _noalloc(lib, B=64, H_q=64, H_kv=8, split=16) == KVC_ERR_WORKSPACE
    assert b"scratch" in lib.kvc_last_error()
    assert _noalloc(lib, H_q=6, H_kv=4) == KVC_ERR_SHAPE
    assert _noalloc(lib, q=None) == KVC_ERR_NULL
    assert _noalloc(lib, B=0) == KVC_OK


def _step_u8(lib, **kw):
    a = dict(B=2, H_q=8, H_kv=2, d=128, q=FAKE, qr=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, T_max=4096, tbl=None,
             bs=0, mb=0, nb=0, pos=FAKE, kn=FAKE, vn=FAKE, cos=FAKE, sin=FAKE, rows=4096, style=0, max_len=4096,
             scale=0.0, out=FAKE, split=0, ws=None, wsn=0, stream=None)
    a.update(kw)
    return lib.kvc_decode_step_u8(a["B"], a["H_q"], a["H_kv"], a["d"], a["q"], a["qr"], a["kc"], a["ks"], a["vc"],
                                  a["vs"], a["T_max"], a["tbl"], a["bs"], a["mb"], a["nb"], a["pos"], a["kn"],
                                  a["vn"], a["cos"], a["sin"], a["rows"], a["style"], a["max_len"], a["scale"],
                                  a["out"], a["split"], a["ws"], a["wsn"], a["stream"])


def test_step_u8_host_checks(lib):
    """The quantized decode step checks its sizes and pointers on the host as
    the quantized decode and the bf16 step do, before anything is launched."""
    assert _step_u8(lib, B=0) == KVC_OK
    assert _step_u8(lib, pos=None) == KVC_ERR_NULL
    assert _step_u8(lib, ks=None) == KVC_ERR_NULL
    assert _step_u8(lib, kn=None) == KVC_ERR_NULL
    assert _step_u8(lib, style=7) == KVC_ERR_UNSUPPORTED
    assert _step_u8(lib, d=96) == KVC_ERR_UNSUPPORTED                 # the kernel's head dims: 64 and 128
    assert _step_u8(lib, H_q=8 * 33, H_kv=8) == KVC_ERR_UNSUPPORTED   # groups of up to 32
    assert _step_u8(lib, max_len=5000) == KVC_ERR_SHAPE               # beyond T_max
    assert _step_u8(lib, tbl=FAKE, bs=8, mb=512, nb=64) == KVC_ERR_UNSUPPORTED   # block size not a multiple of 16
    # a long sequence needs splits: a workspace is required
    need = lib.kvc_decode_workspace_bytes(U8, 2, 8, 2, 128, 100000, 0, 0)
    assert need > 0
    assert _step_u8(lib, T_max=100000, max_len=100000) == KVC_ERR_WORKSPACE


def test_balanced_schedule_choice(lib):
    """The balanced schedule serves ragged paged pools (bf16 or uint8 cache,
    head_dim <= 128, the library's split choice, at most 512 sequences); its
    workspace: the 64 KiB of counters, then two partial rows per query head of
    a group for each of its workgroups (one round: 512 for the bf16 paged
    kernel at head_dim 128 with one 16-head block, two per CU; 768 at head_dim
    64, three per CU; 256 for two 16-head blocks; 512 for the quantized
    kernel's two), or the split plan's size when that is larger."""
    bal = lib.kvc_decode_balanced
    wsb = lib.kvc_decode_workspace_bytes
    zb = lib.kvc_workspace_zeroed_bytes()
    pool = 32 * 8700                                            # ragged paged pool
    assert bal(BF16, 32, 32, 8, 128, 16385, pool, 0) == 1
    assert bal(BF16, 32, 32, 8, 64, 16385, pool, 0) == 1
    assert bal(BF16, 32, 32, 8, 128, 16385, 32 * 16400, 0) == 0  # a pool as large as B * L
    assert bal(BF16, 32, 32, 8, 256, 16385, pool, 0) == 0       # head_dim 256
    assert bal(BF16, 32, 32, 8, 128, 16385, pool, 768) == 0     # explicit splits
    assert bal(F32, 32, 32, 8, 128, 16385, pool, 0) == 0        # the vector kernel
    assert bal(U8, 32, 32, 8, 128, 16385, pool, 0) == 1         # the quantized kernel too
    assert bal(U8, 16, 32, 8, 128, 8193, 0, 0) == 0             # (contiguous: splits)
    assert bal(BF16, 513, 32, 8, 128, 16385, pool, 0) == 0      # more sequences than staged
    assert bal(BF16, 16, 32, 8, 128, 8193, 0, 0) == 0           # contiguous caches: splits
    assert bal(BF16, 64, 32, 1, 128, 4097, 0, 0) == 0
    assert bal(BF16, 16, 30, 8, 128, 100, pool, 0) == -1
    # workspace: the larger of the two layouts
    n = wsb(BF16, 32, 32, 8, 128, 16385, pool, 0)
    assert n >= zb + 512 * 2 * 4 * (8 + 128 * 4) and n % 256 == 0
    assert wsb(BF16, 3, 32, 8, 64, 200, 3 * 16 * 5, 0) == zb + 768 * 2 * 4 * (8 + 64 * 4)
    # groups of 32 heads: 256 workgroups (one per CU), 32 rows each
    assert wsb(BF16, 32, 64, 2, 128, 16385, 32 * 8700, 0) >= zb + 256 * 2 * 32 * (8 + 128 * 4)
    # a short call still needs its partial rows (units shared by workgroups)
    assert wsb(BF16, 3, 32, 8, 128, 200, 3 * 16 * 5, 0) == zb + 512 * 2 * 4 * (8 + 128 * 4)
    assert wsb(U8, 3, 32, 8, 128, 200, 3 * 16 * 5, 0) == zb + 512 * 2 * 4 * (8 + 128 * 4)
