"""C-ABI checks that need no GPU: exported symbols, argument validation, host helpers.

Every rejected call returns its status before any HIP call, so these run on a
machine without a GPU; no call here reaches a kernel launch.
"""

import ctypes
import os
import re

import pytest

import oracle
from bit_quantized_kv_quant_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "minikv.h")

A = 0x10000  # an aligned, never-dereferenced stand-in for a device pointer
MIS = 0x10004  # misaligned stand-in


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(minikv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_header_symbols_exported(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES)


def test_read_probe_validation(L):
    f = L.minikv_read_probe
    assert f(None, 4096, A, None) == -1
    assert f(A, 4096, None, None) == -1
    assert f(A, 0, A, None) == -2
    assert f(A, 4100, A, None) == -2
    assert f(A + 4, 4096, A, None) == -4
    assert f(A, 4096, A + 8, None) == -4


def test_status_strings(L):
    for st in range(0, -7, -1):
        assert _lib.status_string(st)
    assert _lib.status_string(-99) == "unknown status"


def packed(B=1, Hkv=1, n=64, D=128, group=32, ptr=A):
    return _lib.PackedT(ptr, ptr, ptr, ptr, B, Hkv, n, D, group)


def test_prefill_validation(L):
    f = L.minikv_prefill_attn_scores
    args = dict(q=A, k=A, v=A, B=1, T=256, Hq=2, Hkv=2, D=64, W=16, scale=0.0, o=A, lse=A, scores=A)

    def call(**kw):
        a = {**args, **kw}
        return f(a["q"], a["k"], a["v"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["W"], a["scale"],
                 a["o"], a["lse"], a["scores"], None)

    assert call(q=None) == _lib.ERR_NULL
    assert call(lse=None) == _lib.ERR_NULL
    assert call(scores=None) == _lib.ERR_NULL
    assert call(B=0) == _lib.ERR_SHAPE
    assert call(Hq=3) == _lib.ERR_SHAPE
    assert call(W=257) == _lib.ERR_SHAPE
    assert call(W=0) == _lib.ERR_SHAPE
    assert call(D=96) == _lib.ERR_UNSUPPORTED
    # one (sequence, head) slice of K / V over 2 GiB (8,388,608 bf16 rows of 128)
    assert call(T=1 << 23, D=128) == _lib.ERR_UNSUPPORTED
    assert L.minikv_window_scores(A, A, A, 1, 1 << 23, 2, 2, 128, 16, 0.0, A, None) == _lib.ERR_UNSUPPORTED
    assert L.minikv_prefill_attn(A, A, A, 1, 1 << 24, 2, 2, 64, 0.0, A, A, None) == _lib.ERR_UNSUPPORTED
    assert call(k=MIS) == _lib.ERR_ALIGN
    assert call(o=MIS) == _lib.ERR_ALIGN


def test_select_validation(L):
    f = L.minikv_select_topk
    assert f(None, 1, 1, 100, 10, 5, A, None, 0, None) == _lib.ERR_NULL
    assert f(A, 1, 1, 100, 10, 5, None, None, 0, None) == _lib.ERR_NULL
    assert f(A, 1, 1, 100, 90, 11, A, None, 0, None) == _lib.ERR_SHAPE
    assert f(A, 1, 1, 100, -1, 5, A, None, 0, None) == _lib.ERR_SHAPE
    assert f(A, 1, 1, 100, 0, 0, A, None, 0, None) == _lib.ERR_SHAPE
    assert f(A, 1, 1, 70000, 10, 10, A, None, 0, None) == _lib.ERR_UNSUPPORTED
    assert f(MIS, 1, 1, 100, 10, 5, A, None, 0, None) == _lib.ERR_ALIGN
    assert f(A, 1, 1, 100, 10, 5, A, MIS, 64, None) == _lib.ERR_ALIGN     # a workspace, if given, is aligned


def test_select_workspace_size(L):
    """The selection keeps each row on chip: no workspace for any supported row
    length, so NULL / 0 is accepted (the validation above reaches the launch
    stage with ws NULL only on a device)."""
    for B, Hkv, T in [(1, 1, 1), (8, 32, 4096), (1, 32, 16384), (4, 8, 44000), (2, 2, 65536 + 10)]:
        assert L.minikv_select_ws_bytes(B, Hkv, T) == 0
    assert L.minikv_select_ws_bytes(0, 1, 1) == 0


def test_build_id_matches_sources(L):
    """The loaded library reports the hash of the sources it was built from,
    and the loader has checked it against the sources in the tree."""
    from bit_quantized_kv_quant_amd import build

    bid = L.minikv_build_id().decode()
    assert re.fullmatch(r"sha256:[0-9a-f]{16}", bid)
    assert bid == build.source_hash()


def test_stream_init_validation(L):
    f = L.minikv_stream_init
    npk, nres = ctypes.c_int(-7), ctypes.c_int(-7)
    ok = dict(k=A, v=A, idx=A, B=2, Hkv=4, T=256, D=128, n=100, cap=128, kc=A, ks=A, vc=A, vs=A, kr=A, vr=A,
              np_=ctypes.byref(npk), nr=ctypes.byref(nres))

    def call(**kw):
        a = {**ok, **kw}
        return f(a["k"], a["v"], a["idx"], a["B"], a["Hkv"], a["T"], a["D"], a["n"], a["cap"], a["kc"], a["ks"],
                 a["vc"], a["vs"], a["kr"], a["vr"], a["np_"], a["nr"], None)

    assert call(idx=None) == _lib.ERR_NULL
    assert call(vr=None) == _lib.ERR_NULL
    assert call(np_=None) == _lib.ERR_NULL
    assert call(n=0) == _lib.ERR_SHAPE
    assert call(n=257) == _lib.ERR_SHAPE           # more kept tokens than the context
    assert call(cap=100) == _lib.ERR_SHAPE         # capacity not whole groups
    assert call(cap=64) == _lib.ERR_SHAPE          # 96 packed tokens do not fit 64
    assert call(n=127, cap=64) == _lib.ERR_SHAPE   # 96 packed + 31 in the window: too many
    assert call(D=96) == _lib.ERR_UNSUPPORTED
    assert call(T=1 << 23) == _lib.ERR_UNSUPPORTED  # a bf16 K / V slice over 2 GiB
    assert call(kr=MIS) == _lib.ERR_ALIGN
    assert (npk.value, nres.value) == (-7, -7)     # rejected calls leave the counts alone


def test_stream_append_token_validation(L):
    """Counts out of range, and a token that would fill the window with no room
    left to pack it, are rejected before anything is enqueued."""
    f = L.minikv_stream_append_token

    def call(n_packed, n_res, cap=128, D=128, kn=A, kr=A):
        a, b = ctypes.c_int(n_packed), ctypes.c_int(n_res)
        st = f(kn, A, 2, 4, D, cap, ctypes.byref(a), ctypes.byref(b), A, A, A, A, kr, A, None)
        assert (a.value, b.value) == (n_packed, n_res)
        return st

    assert call(0, 0, kn=None) == _lib.ERR_NULL
    assert f(A, A, 2, 4, 128, 128, None, None, A, A, A, A, A, A, None) == _lib.ERR_NULL
    assert call(16, 0) == _lib.ERR_SHAPE           # packed count not whole groups
    assert call(160, 0) == _lib.ERR_SHAPE          # packed count past the capacity
    assert call(0, 32) == _lib.ERR_SHAPE           # a window holds at most 31
    assert call(0, -1) == _lib.ERR_SHAPE
    assert call(128, 31) == _lib.ERR_SHAPE         # the 32nd token cannot be packed: full
    assert call(96, 31, D=96) == _lib.ERR_UNSUPPORTED
    assert call(96, 31, kr=MIS) == _lib.ERR_ALIGN


def test_quant_pack_validation(L):
    f = L.minikv_quant_pack
    p = packed(n=64, D=128)
    byref = ctypes.byref
    assert f(None, A, _lib.BF16, A, 1, 1, 256, 128, 64, byref(p), None) == _lib.ERR_NULL
    assert f(A, A, _lib.BF16, A, 1, 1, 256, 128, 64, None, None) == _lib.ERR_NULL
    pn = packed(ptr=None)
    assert f(A, A, _lib.BF16, A, 1, 1, 256, 128, 64, byref(pn), None) == _lib.ERR_NULL
    assert f(A, A, _lib.BF16, A, 1, 1, 32, 128, 64, byref(p), None) == _lib.ERR_SHAPE     # n_keep > T
    assert f(A, A, _lib.BF16, A, 2, 1, 256, 128, 64, byref(p), None) == _lib.ERR_SHAPE    # B mismatch
    assert f(A, A, _lib.BF16, None, 1, 1, 256, 128, 64, byref(p), None) == _lib.ERR_SHAPE  # idx NULL, n != T
    p96 = packed(D=96)
    assert f(A, A, _lib.BF16, A, 1, 1, 256, 96, 64, byref(p96), None) == _lib.ERR_UNSUPPORTED
    pg = packed(group=16)
    assert f(A, A, _lib.BF16, A, 1, 1, 256, 128, 64, byref(pg), None) == _lib.ERR_UNSUPPORTED
    assert f(A, A, 7, A, 1, 1, 256, 128, 64, byref(p), None) == _lib.ERR_UNSUPPORTED
    assert f(A, MIS, _lib.BF16, A, 1, 1, 256, 128, 64, byref(p), None) == _lib.ERR_ALIGN
    pm = packed(ptr=MIS)
    assert f(A, A, _lib.BF16, A, 1, 1, 256, 128, 64, byref(pm), None) == _lib.ERR_ALIGN
    # a K / V slice over 2 GiB: 4,194,304 fp32 rows or 8,388,608 bf16 rows of 128
    assert f(A, A, _lib.F32, A, 1, 1, 1 << 22, 128, 64, byref(p), None) == _lib.ERR_UNSUPPORTED
    assert f(A, A, _lib.BF16, A, 1, 1, 1 << 23, 128, 64, byref(p), None) == _lib.ERR_UNSUPPORTED


def test_decode_validation(L):
    f = L.minikv_decode_attn
    byref = ctypes.byref
    p = packed(B=2, Hkv=4, n=100, D=128)
    need = L.minikv_decode_ws_bytes(2, 8, 4, 100, 128)
    assert need > 0
    assert f(None, byref(p), 8, 0.0, A, A, need, None) == _lib.ERR_NULL
    assert f(A, None, 8, 0.0, A, A, need, None) == _lib.ERR_NULL
    assert f(A, byref(p), 8, 0.0, None, A, need, None) == _lib.ERR_NULL
    assert f(A, byref(p), 6, 0.0, A, A, need, None) == _lib.ERR_SHAPE    # Hq % Hkv
    assert f(A, byref(p), 32, 0.0, A, A, need, None) == _lib.ERR_UNSUPPORTED  # 8 query heads per KV head
    p64 = packed(B=2, Hkv=4, n=100, D=96)
    assert f(A, byref(p64), 8, 0.0, A, A, need, None) == _lib.ERR_UNSUPPORTED
    assert f(MIS, byref(p), 8, 0.0, A, A, need, None) == _lib.ERR_ALIGN
    assert f(A, byref(p), 8, 0.0, A, A, need - 4, None) == _lib.ERR_WORKSPACE
    assert f(A, byref(p), 8, 0.0, A, None, need, None) == _lib.ERR_WORKSPACE


def test_stream_pack_validation(L):
    f = L.minikv_stream_pack
    ok = (A, A, _lib.BF16, A, 96, 2, 4, 256, 128, 64, 128, 32, A, A, A, A, None)
    args = list(ok)

    def call(**kw):
        a = list(ok)
        pos = {"k": 0, "idx": 3, "idx_stride": 4, "T": 7, "D": 8, "n": 9, "cap": 10, "tok0": 11, "k_codes": 12,
               "dtype": 2}
        for name, val in kw.items():
            a[pos[name]] = val
        return f(*a)

    assert call(k=None) == _lib.ERR_NULL
    assert call(k_codes=None) == _lib.ERR_NULL
    assert call(n=48) == _lib.ERR_SHAPE          # not whole groups
    assert call(tok0=16) == _lib.ERR_SHAPE       # not on a group boundary
    assert call(cap=80) == _lib.ERR_SHAPE        # capacity not whole groups
    assert call(tok0=96) == _lib.ERR_SHAPE       # 96 + 64 > 128
    assert call(idx_stride=32) == _lib.ERR_SHAPE  # index rows shorter than n
    assert call(idx=None, T=32) == _lib.ERR_SHAPE  # identity rows beyond T
    assert call(D=96) == _lib.ERR_UNSUPPORTED
    assert call(dtype=7) == _lib.ERR_UNSUPPORTED
    assert call(T=1 << 23) == _lib.ERR_UNSUPPORTED                 # bf16 K / V slice over 2 GiB
    assert call(T=1 << 22, dtype=_lib.F32) == _lib.ERR_UNSUPPORTED  # fp32 likewise
    assert call(k=MIS) == _lib.ERR_ALIGN
    assert call(k_codes=MIS) == _lib.ERR_ALIGN
    assert len(args) == 17


def test_stream_append_validation(L):
    f = L.minikv_stream_append
    assert f(None, A, None, 1, 2, 4, 1, 128, 1, 0, A, A, None) == _lib.ERR_NULL
    assert f(A, A, None, 1, 2, 4, 1, 128, 1, 0, None, A, None) == _lib.ERR_NULL
    assert f(A, A, None, 1, 2, 4, 1, 128, 1, 32, A, A, None) == _lib.ERR_SHAPE   # slot past the window
    assert f(A, A, A, 20, 2, 4, 600, 128, 8, 28, A, A, None) == _lib.ERR_SHAPE   # 28 + 8 > 32
    assert f(A, A, A, 4, 2, 4, 600, 128, 8, 0, A, A, None) == _lib.ERR_SHAPE     # idx stride < n
    assert f(A, A, None, 1, 2, 4, 1, 128, 2, 0, A, A, None) == _lib.ERR_SHAPE    # 2 rows of a 1-row source
    assert f(A, A, None, 1, 2, 4, 1, 96, 1, 0, A, A, None) == _lib.ERR_UNSUPPORTED
    assert f(A, A, A, 8, 2, 4, 1 << 23, 128, 8, 0, A, A, None) == _lib.ERR_UNSUPPORTED  # K / V slice over 2 GiB
    assert f(A, MIS, None, 1, 2, 4, 1, 128, 1, 0, A, A, None) == _lib.ERR_ALIGN


def test_stream_decode_validation(L):
    f = L.minikv_stream_decode
    need = L.minikv_stream_decode_ws_bytes(2, 8, 4, 64, 5, 128)
    assert need > 0
    assert L.minikv_stream_decode_ws_bytes(2, 8, 4, 48, 5, 128) == 0   # packed tokens not whole groups
    assert L.minikv_stream_decode_ws_bytes(2, 8, 4, 64, 32, 128) == 0  # residual holds at most 31
    assert L.minikv_stream_decode_ws_bytes(2, 8, 4, 0, 0, 128) == 0    # nothing to attend

    def call(q=A, Hq=8, cap=128, n_packed=64, k_codes=A, k_res=A, n_res=5, out=A, ws=A, ws_bytes=need, D=128):
        return f(q, 2, Hq, 4, D, cap, n_packed, k_codes, A, A, A, k_res, A, n_res, 0.0, out, ws, ws_bytes, None)

    assert call(q=None) == _lib.ERR_NULL
    assert call(k_codes=None) == _lib.ERR_NULL
    assert call(k_res=None) == _lib.ERR_NULL
    assert call(Hq=6) == _lib.ERR_SHAPE
    assert call(n_packed=48) == _lib.ERR_SHAPE
    assert call(n_packed=160) == _lib.ERR_SHAPE      # beyond the capacity
    assert call(n_res=32) == _lib.ERR_SHAPE
    assert call(n_packed=0, n_res=0) == _lib.ERR_SHAPE
    assert call(cap=100) == _lib.ERR_SHAPE
    assert call(Hq=32) == _lib.ERR_UNSUPPORTED        # 8 query heads per KV head
    assert call(D=96) == _lib.ERR_UNSUPPORTED
    assert call(q=MIS) == _lib.ERR_ALIGN
    assert call(k_res=MIS) == _lib.ERR_ALIGN
    assert call(ws_bytes=need - 4) == _lib.ERR_WORKSPACE
    assert call(ws=None) == _lib.ERR_WORKSPACE


def test_device_step_validation(L):
    sc = L.minikv_stream_set_counts
    assert sc(None, 0, 0, 64, None) == _lib.ERR_NULL
    assert sc(A, 16, 0, 64, None) == _lib.ERR_SHAPE      # packed tokens not whole groups
    assert sc(A, 96, 0, 64, None) == _lib.ERR_SHAPE      # beyond the capacity
    assert sc(A, 0, 32, 64, None) == _lib.ERR_SHAPE      # the window holds at most 31
    assert sc(A, 0, 0, 48, None) == _lib.ERR_SHAPE       # capacity not whole groups
    assert sc(MIS, 0, 0, 64, None) == _lib.ERR_ALIGN

    ap = L.minikv_stream_step_append

    def app(k=A, B=2, D=128, cap=128, counts=A, k_res=A):
        return ap(k, A, B, 4, D, cap, counts, A, A, A, A, k_res, A, None)

    assert app(k=None) == _lib.ERR_NULL
    assert app(counts=None) == _lib.ERR_NULL
    assert app(k_res=None) == _lib.ERR_NULL
    assert app(B=0) == _lib.ERR_SHAPE
    assert app(cap=100) == _lib.ERR_SHAPE
    assert app(D=96) == _lib.ERR_UNSUPPORTED
    assert app(counts=MIS) == _lib.ERR_ALIGN

    need = L.minikv_stream_step_decode_ws_bytes(2, 8, 4, 128, 128)
    assert need > 0
    assert L.minikv_stream_step_decode_ws_bytes(2, 8, 3, 128, 128) == 0
    assert L.minikv_stream_step_decode_ws_bytes(2, 8, 4, 100, 128) == 0
    # planned for the whole capacity, with a window part: at least the host-count workspace
    assert need >= L.minikv_stream_decode_ws_bytes(2, 8, 4, 128, 31, 128)
    f = L.minikv_stream_step_decode

    def dec(q=A, Hq=8, cap=128, counts=A, ws=A, ws_bytes=need, D=128):
        return f(q, 2, Hq, 4, D, cap, counts, A, A, A, A, A, A, 0.0, A, ws, ws_bytes, None)

    assert dec(q=None) == _lib.ERR_NULL
    assert dec(counts=None) == _lib.ERR_NULL
    assert dec(ws=None) == _lib.ERR_NULL
    assert dec(Hq=6) == _lib.ERR_SHAPE
    assert dec(cap=100) == _lib.ERR_SHAPE
    assert dec(Hq=32) == _lib.ERR_UNSUPPORTED
    assert dec(D=96) == _lib.ERR_UNSUPPORTED
    assert dec(counts=MIS) == _lib.ERR_ALIGN
    assert dec(ws_bytes=need - 4) == _lib.ERR_WORKSPACE


def test_host_budget_helpers_match_oracle(L):
    for T in (1, 7, 256, 4096, 8192, 16384, 44000, 65536):
        for pct in (5, 15, 30, 100):
            assert L.minikv_keep_count(T, pct * 1000) == oracle.keep_count(T, pct)
    for L_ in (1, 2, 32, 40):
        for layer in range(L_):
            assert L.minikv_pyramid_keep(8192, L_, layer, 30, 5) == oracle.pyramid_keep(8192, L_, layer)
    h, r = ctypes.c_int(), ctypes.c_int()
    for n in (1, 4, 5, 64, 614, 2457, 6600):
        assert L.minikv_split_heavy_recent(n, h, r) == 0
        assert (h.value, r.value) == oracle.split_heavy_recent(n)
    assert L.minikv_keep_count(0, 15000) == _lib.ERR_SHAPE
    assert L.minikv_pyramid_keep(100, 4, 4, 30, 5) == _lib.ERR_SHAPE


def test_packed_bytes_matches_oracle(L):
    for n in (1, 31, 32, 33, 64, 614, 2457, 6600):
        for D in (64, 128):
            assert L.minikv_packed_bytes(3, 5, n, D) == oracle.packed_bytes_ref(3, 5, n, D)
    assert L.minikv_packed_bytes(0, 1, 1, 128) == 0


def test_single_pass_rule(L):
    """Scores come out of pass 1 exactly for one query head per KV head, W <= 32,
    W rows inside the last 256-row query block and at least one head per
    compute unit (256 assumed without a device); invalid sizes give 0."""
    f = L.minikv_prefill_fuses_scores
    assert f(8, 4096, 32, 32, 32) == 1
    assert f(1, 16384, 32, 32, 32) == 0         # 32 heads: the stand-alone pass is faster
    assert f(256, 1, 1, 1, 1) == 1
    assert f(4, 44000, 32, 8, 32) == 0          # four query heads per KV head
    assert f(8, 4096, 32, 32, 33) == 0          # window beyond one row block
    assert f(16, 4100, 16, 16, 4) == 1          # last block holds rows 4096..4099
    assert f(16, 4100, 16, 16, 5) == 0
    for T in (1, 255, 256, 257, 511, 44000):
        last = T - (T - 1) // 256 * 256
        for W in (1, 16, 32):
            assert f(64, T, 4, 4, W) == int(W <= min(32, last, T))
    assert f(0, 10, 1, 1, 1) == 0 and f(1, 10, 3, 2, 1) == 0 and f(1, 10, 1, 1, 11) == 0


def test_decode_noalloc_validation(L):
    """Argument checks of the allocation-free decode (no HIP call is reached)."""
    f = L.minikv_decode_attn_noalloc
    byref = ctypes.byref
    p = packed(B=2, Hkv=4, n=100, D=128)
    assert f(None, byref(p), 8, 0.0, A, None) == _lib.ERR_NULL
    assert f(A, None, 8, 0.0, A, None) == _lib.ERR_NULL
    assert f(A, byref(p), 8, 0.0, None, None) == _lib.ERR_NULL
    assert f(A, byref(packed(ptr=None)), 8, 0.0, A, None) == _lib.ERR_NULL
    assert f(A, byref(p), 6, 0.0, A, None) == _lib.ERR_SHAPE
    assert f(A, byref(p), 32, 0.0, A, None) == _lib.ERR_UNSUPPORTED
    assert f(A, byref(packed(B=2, Hkv=4, n=100, D=96)), 8, 0.0, A, None) == _lib.ERR_UNSUPPORTED
    assert f(A, byref(packed(group=16)), 1, 0.0, A, None) == _lib.ERR_UNSUPPORTED
    assert f(MIS, byref(p), 8, 0.0, A, None) == _lib.ERR_ALIGN
    assert f(A, byref(p), 8, 0.0, MIS, None) == _lib.ERR_ALIGN


def test_every_decode_split_plan_fits_the_scratch_array(L):
    """The decode workspace of any supported shape - the 16 KiB ticket area,
    then one part of D + 2 floats per query head and token range (merged by
    the merge kernel) or per workgroup of four ranges after a head's first
    (merged inside the launch) - fits the allocation-free entry point's array:
    (sequence, KV head) units x parts stay below 8192 (one range per head, or
    one workgroup, needs no parts)."""
    worst = 0
    for units in list(range(1, 300)) + list(range(300, 4200, 7)) + [4095, 4096, 5000, 20000]:
        for n in (1, 129, 614, 6600, 65536, 1 << 20):
            for R in (1, 2, 4):
                for D in (64, 128):
                    ws = L.minikv_decode_ws_bytes(units, R, 1, n, D)
                    assert ws >= _lib.DECODE_TICKET_BYTES
                    parts = (ws - _lib.DECODE_TICKET_BYTES) // (units * R * (D + 2) * 4)
                    assert parts * units * R * (D + 2) * 4 + _lib.DECODE_TICKET_BYTES == ws
                    if units >= 4096 or n <= 128:
                        assert parts == 0           # one range per head: the output is written directly
                    assert units * parts < 8192
                    worst = max(worst, ws)
    assert worst <= _lib.DECODE_SCRATCH_BYTES
    print("largest decode workspace:", worst)
