"""Torch-facing wrappers of the C ABI (include/minikv.h).

Tensors are torch CUDA (HIP) tensors used as device memory; each wrapper checks
dtypes / shapes / contiguity, allocates outputs when none are given, and calls
the library on the current torch stream.  No arithmetic of the method happens
here.
"""

import ctypes
from dataclasses import dataclass

import torch

from . import _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


@dataclass
class PackedCache:
    """Packed 2-bit cache (layout of minikv_packed_t) held in torch tensors."""

    k_codes: torch.Tensor  # uint8 [B, Hkv, n, D/4]
    k_sz: torch.Tensor     # int32 bits of (fp16 s | fp16 z << 16) [B, Hkv, ceil(n/32), D]
    v_codes: torch.Tensor  # uint8 [B, Hkv, ceil(n/32), D, 8]: 32 tokens of a channel per 8 bytes
    v_sz: torch.Tensor     # int32 [B, Hkv, n, D/32]
    B: int
    Hkv: int
    n_keep: int
    D: int

    @staticmethod
    def alloc(B, Hkv, n_keep, D, device="cuda"):
        G = -(-n_keep // _lib.GROUP)
        return PackedCache(
            torch.empty((B, Hkv, n_keep, D // 4), dtype=torch.uint8, device=device),
            torch.empty((B, Hkv, G, D), dtype=torch.int32, device=device),
            torch.empty((B, Hkv, G, D, 8), dtype=torch.uint8, device=device),
            torch.empty((B, Hkv, n_keep, D // _lib.GROUP), dtype=torch.int32, device=device),
            B, Hkv, n_keep, D)

    def struct(self):
        return _lib.PackedT(self.k_codes.data_ptr(), self.k_sz.data_ptr(), self.v_codes.data_ptr(),
                            self.v_sz.data_ptr(), self.B, self.Hkv, self.n_keep, self.D, _lib.GROUP)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in (self.k_codes, self.k_sz, self.v_codes, self.v_sz))


def _check_qkv(q, k, v):
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    _need(q, torch.bfloat16, (B, Hq, T, D), "q")
    _need(k, torch.bfloat16, (B, Hkv, T, D), "k")
    if v is not None:
        _need(v, torch.bfloat16, (B, Hkv, T, D), "v")
    return B, Hq, Hkv, T, D


def prefill_attn(q, k, v, sm_scale=None, with_o=True, o=None, lse=None):
    """Pass 1: causal attention o (bf16, or None) and per-row lse (fp32)."""
    B, Hq, Hkv, T, D = _check_qkv(q, k, v)
    if with_o and o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if o is not None:
        _need(o, torch.bfloat16, (B, Hq, T, D), "o")
    _need(lse, torch.float32, (B, Hq, T), "lse")
    st = _lib.lib().minikv_prefill_attn(_ptr(q), _ptr(k), _ptr(v), B, T, Hq, Hkv, D, float(sm_scale or 0.0),
                                        _ptr(o) if o is not None else None, _ptr(lse), _stream())
    _lib.check("minikv_prefill_attn", st)
    return o, lse


def window_scores(q, k, lse, window, sm_scale=None, scores=None):
    """Pass 2 (the second kernel): per-key probability mass from the last `window` rows."""
    B, Hq, Hkv, T, D = _check_qkv(q, k, None)
    _need(lse, torch.float32, (B, Hq, T), "lse")
    if scores is None:
        scores = torch.empty((B, Hkv, T), dtype=torch.float32, device=q.device)
    _need(scores, torch.float32, (B, Hkv, T), "scores")
    st = _lib.lib().minikv_window_scores(_ptr(q), _ptr(k), _ptr(lse), B, T, Hq, Hkv, D, int(window),
                                         float(sm_scale or 0.0), _ptr(scores), _stream())
    _lib.check("minikv_window_scores", st)
    return scores


def prefill_attn_scores(q, k, v, window, sm_scale=None, with_o=True, o=None, lse=None, scores=None):
    """Both passes of selective flash attention: returns (o or None, lse, scores)."""
    B, Hq, Hkv, T, D = _check_qkv(q, k, v)
    if with_o and o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if scores is None:
        scores = torch.empty((B, Hkv, T), dtype=torch.float32, device=q.device)
    if o is not None:
        _need(o, torch.bfloat16, (B, Hq, T, D), "o")
    _need(lse, torch.float32, (B, Hq, T), "lse")
    _need(scores, torch.float32, (B, Hkv, T), "scores")
    st = _lib.lib().minikv_prefill_attn_scores(
        _ptr(q), _ptr(k), _ptr(v), B, T, Hq, Hkv, D, int(window), float(sm_scale or 0.0),
        _ptr(o) if o is not None else None, _ptr(lse), _ptr(scores), _stream())
    _lib.check("minikv_prefill_attn_scores", st)
    return o, lse, scores


def prefill_fuses_scores(B, T, Hq, Hkv, window):
    """True where prefill_attn_scores runs as one launch (scores from inside pass 1)."""
    return bool(_lib.lib().minikv_prefill_fuses_scores(int(B), int(T), int(Hq), int(Hkv), int(window)))


def select_ws_bytes(B, Hkv, T):
    return int(_lib.lib().minikv_select_ws_bytes(int(B), int(Hkv), int(T)))


def select_topk(scores, n_heavy, n_recent, idx=None, ws=None):
    """Heavy-hitter + recent selection: scores fp32 [B, Hkv, T] -> idx int32 [B, Hkv, n], ascending."""
    B, Hkv, T = scores.shape
    _need(scores, torch.float32, (B, Hkv, T), "scores")
    n = n_heavy + n_recent
    if idx is None:
        idx = torch.empty((B, Hkv, n), dtype=torch.int32, device=scores.device)
    _need(idx, torch.int32, (B, Hkv, n), "idx")
    need = select_ws_bytes(B, Hkv, T)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = _lib.lib().minikv_select_topk(_ptr(scores), B, Hkv, T, int(n_heavy), int(n_recent), _ptr(idx), _ptr(ws),
                                       ws_bytes, _stream())
    _lib.check("minikv_select_topk", st)
    return idx


def quant_pack(k, v, idx=None, out=None):
    """Quantise / pack the kept tokens of fp32 or bf16 k, v [B, Hkv, T, D]."""
    B, Hkv, T, D = k.shape
    if k.dtype == torch.float32:
        dt = _lib.F32
    elif k.dtype == torch.bfloat16:
        dt = _lib.BF16
    else:
        raise TypeError("k, v must be fp32 or bf16")
    _need(k, k.dtype, (B, Hkv, T, D), "k")
    _need(v, k.dtype, (B, Hkv, T, D), "v")
    n = T if idx is None else idx.shape[-1]
    if idx is not None:
        _need(idx, torch.int32, (B, Hkv, n), "idx")
    if out is None:
        out = PackedCache.alloc(B, Hkv, n, D, k.device)
    s = out.struct()
    st = _lib.lib().minikv_quant_pack(_ptr(k), _ptr(v), dt, _ptr(idx) if idx is not None else None,
                                      B, Hkv, T, D, n, ctypes.byref(s), _stream())
    _lib.check("minikv_quant_pack", st)
    return out


def decode_ws_bytes(B, Hq, Hkv, n_keep, D):
    return int(_lib.lib().minikv_decode_ws_bytes(B, Hq, Hkv, n_keep, D))


def decode_attn(q, cache, sm_scale=None, out=None, ws=None):
    """Single-query attention over the packed cache: q bf16 [B, Hq, D] -> bf16 [B, Hq, D]."""
    B, Hq, D = q.shape
    _need(q, torch.bfloat16, (B, Hq, D), "q")
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, (B, Hq, D), "out")
    need = decode_ws_bytes(B, Hq, cache.Hkv, cache.n_keep, D)
    if ws is None:
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    s = cache.struct()
    st = _lib.lib().minikv_decode_attn(_ptr(q), ctypes.byref(s), Hq, float(sm_scale or 0.0), _ptr(out),
                                       _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _lib.check("minikv_decode_attn", st)
    return out


@dataclass
class StreamCache:
    """Streaming cache: a packed region laid out for `cap` tokens (whole 32-token
    groups; the first n_packed are valid) and a bf16 residual window of 32 slots
    per (sequence, KV head) (the first n_res are valid).  Generated tokens are
    appended to the window; 32 of them are packed as the next group."""

    k_codes: torch.Tensor  # uint8 [B, Hkv, cap, D/4]
    k_sz: torch.Tensor     # int32 [B, Hkv, cap/32, D]
    v_codes: torch.Tensor  # uint8 [B, Hkv, cap/32, D, 8]
    v_sz: torch.Tensor     # int32 [B, Hkv, cap, D/32]
    k_res: torch.Tensor    # bf16 [B, Hkv, 32, D]
    v_res: torch.Tensor    # bf16 [B, Hkv, 32, D]
    B: int
    Hkv: int
    cap: int
    D: int
    n_packed: int = 0
    n_res: int = 0
    counts: torch.Tensor = None  # int32 [4] {n_packed, n_res, overflow, ticket}: the device-side step's counts

    @staticmethod
    def alloc(B, Hkv, cap, D, device="cuda"):
        if cap < _lib.GROUP or cap % _lib.GROUP:
            raise ValueError("cap must be a positive multiple of 32")
        G = cap // _lib.GROUP
        return StreamCache(
            torch.empty((B, Hkv, cap, D // 4), dtype=torch.uint8, device=device),
            torch.empty((B, Hkv, G, D), dtype=torch.int32, device=device),
            torch.empty((B, Hkv, G, D, 8), dtype=torch.uint8, device=device),
            torch.empty((B, Hkv, cap, D // _lib.GROUP), dtype=torch.int32, device=device),
            torch.empty((B, Hkv, _lib.GROUP, D), dtype=torch.bfloat16, device=device),
            torch.empty((B, Hkv, _lib.GROUP, D), dtype=torch.bfloat16, device=device),
            B, Hkv, cap, D)

    def _bufs(self):
        return (_ptr(self.k_codes), _ptr(self.k_sz), _ptr(self.v_codes), _ptr(self.v_sz), _ptr(self.k_res),
                _ptr(self.v_res))

    def init(self, k, v, idx):
        """Start from a selection idx int32 [B, Hkv, n] of bf16 k, v [B, Hkv, T, D]:
        the library packs its whole groups and puts the rest in the window."""
        B, Hkv, T, D = k.shape
        _need(k, torch.bfloat16, (self.B, self.Hkv, T, self.D), "k")
        _need(v, torch.bfloat16, (self.B, self.Hkv, T, self.D), "v")
        n = idx.shape[-1]
        _need(idx, torch.int32, (self.B, self.Hkv, n), "idx")
        n_packed, n_res = ctypes.c_int(self.n_packed), ctypes.c_int(self.n_res)
        kc, ks, vc, vs, kr, vr = self._bufs()
        st = _lib.lib().minikv_stream_init(_ptr(k), _ptr(v), _ptr(idx), self.B, self.Hkv, int(T), self.D, int(n),
                                           self.cap, kc, ks, vc, vs, kr, vr, ctypes.byref(n_packed),
                                           ctypes.byref(n_res), _stream())
        _lib.check("minikv_stream_init", st)
        self.n_packed, self.n_res = n_packed.value, n_res.value
        return self

    def append(self, k_new, v_new):
        """One generated token per (sequence, KV head): k_new, v_new bf16 [B, Hkv, D].
        The library packs the window as the next group when the token fills it
        (a full cache raises MinikvError with the shape status)."""
        _need(k_new, torch.bfloat16, (self.B, self.Hkv, self.D), "k_new")
        _need(v_new, torch.bfloat16, (self.B, self.Hkv, self.D), "v_new")
        n_packed, n_res = ctypes.c_int(self.n_packed), ctypes.c_int(self.n_res)
        kc, ks, vc, vs, kr, vr = self._bufs()
        st = _lib.lib().minikv_stream_append_token(_ptr(k_new), _ptr(v_new), self.B, self.Hkv, self.D, self.cap,
                                                   ctypes.byref(n_packed), ctypes.byref(n_res), kc, ks, vc, vs, kr,
                                                   vr, _stream())
        _lib.check("minikv_stream_append_token", st)
        self.n_packed, self.n_res = n_packed.value, n_res.value
        return self

    def ws_bytes(self, Hq):
        return int(_lib.lib().minikv_stream_decode_ws_bytes(self.B, Hq, self.Hkv, self.n_packed, self.n_res, self.D))

    # ---- device-side generation step: the counts live in device memory, so a
    # step (step_append + step_decode per layer) is a fixed launch sequence that a
    # HIP graph can capture and replay ----

    def to_device_counts(self):
        """Copy the host counts into the device counts (allocated on first use)."""
        if self.counts is None:
            self.counts = torch.empty(4, dtype=torch.int32, device=self.k_res.device)
        st = _lib.lib().minikv_stream_set_counts(_ptr(self.counts), self.n_packed, self.n_res, self.cap, _stream())
        _lib.check("minikv_stream_set_counts", st)
        return self

    def from_device_counts(self):
        """Read the device counts back into n_packed / n_res (synchronises); raises on overflow."""
        n_packed, n_res, overflow, _ = (int(x) for x in self.counts.cpu())
        if overflow:
            raise ValueError("streaming cache is full (a window could not be packed)")
        self.n_packed, self.n_res = n_packed, n_res
        return self

    def step_append(self, k_new, v_new):
        """append() with the counts on the device (no host decision)."""
        if self.counts is None:
            raise ValueError("call to_device_counts() first")
        _need(k_new, torch.bfloat16, (self.B, self.Hkv, self.D), "k_new")
        _need(v_new, torch.bfloat16, (self.B, self.Hkv, self.D), "v_new")
        st = _lib.lib().minikv_stream_step_append(_ptr(k_new), _ptr(v_new), self.B, self.Hkv, self.D, self.cap,
                                                  _ptr(self.counts), _ptr(self.k_codes), _ptr(self.k_sz),
                                                  _ptr(self.v_codes), _ptr(self.v_sz), _ptr(self.k_res),
                                                  _ptr(self.v_res), _stream())
        _lib.check("minikv_stream_step_append", st)
        return self

    def step_ws_bytes(self, Hq):
        return int(_lib.lib().minikv_stream_step_decode_ws_bytes(self.B, Hq, self.Hkv, self.cap, self.D))

    def step_decode(self, q, sm_scale=None, out=None, ws=None):
        """decode() with the counts read on the device."""
        if self.counts is None:
            raise ValueError("call to_device_counts() first")
        B, Hq, D = q.shape
        _need(q, torch.bfloat16, (self.B, Hq, self.D), "q")
        if out is None:
            out = torch.empty_like(q)
        _need(out, torch.bfloat16, (self.B, Hq, self.D), "out")
        if ws is None:
            ws = torch.zeros(max(self.step_ws_bytes(Hq), 16), dtype=torch.uint8, device=q.device)
        st = _lib.lib().minikv_stream_step_decode(_ptr(q), self.B, Hq, self.Hkv, self.D, self.cap, _ptr(self.counts),
                                                  _ptr(self.k_codes), _ptr(self.k_sz), _ptr(self.v_codes),
                                                  _ptr(self.v_sz), _ptr(self.k_res), _ptr(self.v_res),
                                                  float(sm_scale or 0.0), _ptr(out), _ptr(ws),
                                                  ws.numel() * ws.element_size(), _stream())
        _lib.check("minikv_stream_step_decode", st)
        return out

    def decode(self, q, sm_scale=None, out=None, ws=None):
        """Single-query attention over the packed and the residual tokens: q bf16 [B, Hq, D]."""
        B, Hq, D = q.shape
        _need(q, torch.bfloat16, (self.B, Hq, self.D), "q")
        if out is None:
            out = torch.empty_like(q)
        _need(out, torch.bfloat16, (self.B, Hq, self.D), "out")
        need = self.ws_bytes(Hq)
        if ws is None:
            ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
        st = _lib.lib().minikv_stream_decode(_ptr(q), self.B, Hq, self.Hkv, self.D, self.cap, self.n_packed,
                                             _ptr(self.k_codes), _ptr(self.k_sz), _ptr(self.v_codes),
                                             _ptr(self.v_sz), _ptr(self.k_res), _ptr(self.v_res), self.n_res,
                                             float(sm_scale or 0.0), _ptr(out), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream())
        _lib.check("minikv_stream_decode", st)
        return out


READ_PROBE_SINK_WORDS = 131072  # MINIKV_READ_PROBE_SINK_WORDS: one word per wave of the probe's grid


def read_probe(x, sink=None):
    """Streaming read of the bytes of a contiguous device tensor (a measurement aid,
    not a step of the method): returns the int32 sink, whose XOR is the XOR of
    every 32-bit word of x."""
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    if sink is None:
        sink = torch.zeros(READ_PROBE_SINK_WORDS, dtype=torch.int32, device=x.device)
    _need(sink, torch.int32, (READ_PROBE_SINK_WORDS,), "sink")
    st = _lib.lib().minikv_read_probe(_ptr(x), x.numel() * x.element_size(), _ptr(sink), _stream())
    _lib.check("minikv_read_probe", st)
    return sink


def packed_bytes(B, Hkv, n_keep, D):
    return int(_lib.lib().minikv_packed_bytes(B, Hkv, n_keep, D))


def keep_count(T, pct):
    r = _lib.lib().minikv_keep_count(int(T), int(round(pct * 1000)))
    _lib.check("minikv_keep_count", 0 if r > 0 else r)
    return r


def pyramid_keep(T, n_layers, layer, first_pct=30, last_pct=5):
    r = _lib.lib().minikv_pyramid_keep(int(T), int(n_layers), int(layer), int(first_pct), int(last_pct))
    _lib.check("minikv_pyramid_keep", 0 if r > 0 else r)
    return r


def split_heavy_recent(n_keep):
    h, r = ctypes.c_int(), ctypes.c_int()
    _lib.check("minikv_split_heavy_recent", _lib.lib().minikv_split_heavy_recent(int(n_keep), h, r))
    return h.value, r.value
