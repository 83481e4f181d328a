"""Python binding of the verify-step library ``libspecverify.so``.

Argument marshalling only: every step of the verify pass (logits, row
statistics, acceptance, resampling, cache-length commit) runs in the HIP
library behind the C ABI declared in ``include/specverify.h``.  torch supplies
device memory and streams.  The binding fails loudly when the library is
missing or a call returns an error; it has no fallback path.

Functions mirror the C entry points: :func:`verify_forward`,
:func:`spec_verify_greedy`, :func:`spec_verify_sample`, and the drafter's
centroid-masked LM head :func:`draft_masked_logits`.
"""
import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Optional

import torch

__all__ = ["SV_F32", "SV_BF16", "SV_IN_LOGITS", "SV_IN_HIDDEN", "SV_IN_TOKENS", "VerifyError",
           "Model", "KVCache", "Workspace", "lm_head_model", "logits_model", "decoder_model",
           "verify_forward", "spec_verify_greedy", "spec_verify_sample", "spec_verify_sample_noalloc", "library", "library_path",
           "timing_enable", "timing_read", "set_option", "SV_OPT_WAIT_LIMIT", "tune_verify", "LAYER_KEYS", "MaskedHead", "masked_head", "draft_masked_logits"]

SV_F32, SV_BF16 = 0, 1
SV_IN_LOGITS, SV_IN_HIDDEN, SV_IN_TOKENS = 0, 1, 2
LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "libspecverify.so")


class VerifyError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status, name, message):
        super().__init__(f"{name}: {message}")
        self.status = status


class _SvModel(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("wdtype", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("embed", ctypes.c_void_p), ("layers", ctypes.POINTER(ctypes.c_void_p)),
                ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p)]


class _SvMaskedHead(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_clusters", ctypes.c_int32),
                ("wdtype", ctypes.c_int32), ("embed", ctypes.c_void_p), ("centroids", ctypes.c_void_p)]


class _SvDrafter(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("embed", ctypes.c_void_p), ("pre_proj", ctypes.c_void_p),
                ("layers", ctypes.POINTER(ctypes.c_void_p)), ("final_norm", ctypes.c_void_p),
                ("post_proj", ctypes.c_void_p), ("centroids", ctypes.c_void_p), ("n_clusters", ctypes.c_int32),
                ("top_k_clusters", ctypes.c_int32)]


class _SvSharedKV(ctypes.Structure):
    _fields_ = [("k", ctypes.POINTER(ctypes.c_void_p)), ("v", ctypes.POINTER(ctypes.c_void_p)),
                ("max_len", ctypes.c_int32), ("len", ctypes.c_void_p)]


class _SvKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("max_len", ctypes.c_int32),
                ("len", ctypes.c_void_p)]


_lib = None


def library():
    """Load ``libspecverify.so`` (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m accept_step_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)
    M, KV = ctypes.POINTER(_SvModel), ctypes.POINTER(_SvKV)
    lib.verify_forward.argtypes = [M, i32, vp, i32, i32, KV, vp, vp, sz, vp]
    lib.spec_verify_greedy.argtypes = [M, i32, vp, i32, i32, vp, KV, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_sample.argtypes = [M, i32, vp, i32, i32, vp, vp, i32, ctypes.c_float, ctypes.c_uint64, vp,
                                       KV, vp, vp, vp, vp, vp, sz, vp]
    lib.spec_verify_sample_noalloc.argtypes = [M, i32, vp, i32, i32, vp, vp, i32, ctypes.c_float, ctypes.c_uint64,
                                               vp, KV, vp, vp, vp, vp, vp]
    lib.spec_verify_sample_filtered.argtypes = [M, i32, vp, i32, i32, vp, vp, i32, ctypes.c_float, i32,
                                                ctypes.c_float, ctypes.c_uint64, vp, KV, vp, vp, vp, vp, sz, vp]
    lib.draft_masked_logits.argtypes = [ctypes.POINTER(_SvMaskedHead), vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.mtp_draft.argtypes = [ctypes.POINTER(_SvDrafter), ctypes.POINTER(_SvSharedKV), i32, i32, vp, vp,
                              ctypes.c_float, ctypes.c_uint64, vp, vp, i32, vp, sz, vp]
    lib.round_pad_drafts.argtypes = [i32, i32, i32, vp, vp, vp, i32, ctypes.c_float, vp, sz, vp]
    lib.round_update_gamma.argtypes = [i32, vp, vp, i32, i32, vp]
    lib.round_select_candidates.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp]
    for f in (lib.verify_forward, lib.spec_verify_greedy, lib.spec_verify_sample, lib.spec_verify_sample_noalloc,
              lib.sv_timing_enable,
              lib.sv_timing_read, lib.draft_masked_logits, lib.spec_verify_sample_filtered, lib.mtp_draft,
              lib.round_pad_drafts, lib.round_update_gamma, lib.round_select_candidates):
        f.restype = i32
    lib.sv_set_option.argtypes = [i32, ctypes.c_int64]
    lib.sv_set_option.restype = i32
    lib.sv_tune_verify.argtypes = [M, i32, i32, vp]
    lib.sv_tune_verify.restype = i32
    lib.sv_tuned_item.argtypes = [M, i32, i32]
    lib.sv_tuned_item.restype = i32
    lib.sv_version.restype = i32
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_status_string.argtypes = [i32]
    lib.sv_last_error.restype = ctypes.c_char_p
    lib.sv_timing_enable.argtypes = [i32]
    lib.sv_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        lib = library()
        raise VerifyError(status, lib.sv_status_string(status).decode(), lib.sv_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    return t


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Model:
    """A target model for the library: the C struct plus the tensors it points to."""
    struct: _SvModel
    keep: list = field(default_factory=list)
    layer_ptrs: Optional[ctypes.Array] = None

    @property
    def vocab(self):
        return self.struct.vocab


def logits_model(vocab):
    """Model for SV_IN_LOGITS inputs (only the vocabulary size is read)."""
    s = _SvModel()
    s.vocab = int(vocab)
    return Model(s)


def lm_head_model(w):
    """LM-head-only model from a [V, d] bfloat16 or float32 device tensor."""
    _dev_tensor(w, "lm_head")
    s = _SvModel()
    s.n_layers = 0
    s.vocab, s.d_model = int(w.shape[0]), int(w.shape[1])
    if w.dtype == torch.bfloat16:
        s.wdtype = SV_BF16
    elif w.dtype == torch.float32:
        s.wdtype = SV_F32
    else:
        raise ValueError("lm_head must be bfloat16 or float32")
    s.lm_head = w.data_ptr()
    return Model(s, [w])


def decoder_model(embed, layers, final_norm, lm_head, n_heads, head_dim, rms_eps=1e-5, rope_theta=10000.0):
    """Decoder model from bf16 device tensors; ``layers`` is a list of dicts keyed by LAYER_KEYS."""
    keep = [embed, final_norm, lm_head]
    for t, n in ((embed, "embed"), (final_norm, "final_norm"), (lm_head, "lm_head")):
        _dev_tensor(t, n, torch.bfloat16)
    ptrs = (ctypes.c_void_p * (9 * len(layers)))()
    for i, L in enumerate(layers):
        for j, key in enumerate(LAYER_KEYS):
            t = _dev_tensor(L[key], key, torch.bfloat16)
            keep.append(t)
            ptrs[9 * i + j] = t.data_ptr()
    s = _SvModel()
    s.n_layers = len(layers)
    s.d_model = int(embed.shape[1])
    s.n_heads, s.head_dim = int(n_heads), int(head_dim)
    s.d_ff = int(layers[0]["w_gate"].shape[0])
    s.vocab = int(lm_head.shape[0])
    s.wdtype = SV_BF16
    s.rms_eps, s.rope_theta = float(rms_eps), float(rope_theta)
    s.embed, s.final_norm, s.lm_head = embed.data_ptr(), final_norm.data_ptr(), lm_head.data_ptr()
    s.layers = ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p))
    return Model(s, keep, ptrs)


@dataclass
class KVCache:
    """bf16 K/V [n_layers, B, n_heads, max_len, head_dim] and int32 lengths [B]."""
    k: torch.Tensor
    v: torch.Tensor
    length: torch.Tensor

    def struct(self):
        for t, n in ((self.k, "k"), (self.v, "v")):
            _dev_tensor(t, n, torch.bfloat16)
        _dev_tensor(self.length, "length", torch.int32)
        s = _SvKV()
        s.k, s.v = self.k.data_ptr(), self.v.data_ptr()
        s.max_len = int(self.k.shape[3])
        s.len = self.length.data_ptr()
        return s


SV_OPT_WAIT_LIMIT = 0


def set_option(option, value):
    """Process-wide library option (C: sv_set_option); value < 0 restores the default."""
    _check(library().sv_set_option(int(option), int(value)))


def tune_verify(model, B, gamma, stream=None):
    """Choose the fused step's load grouping for this device and shape (C:
    sv_tune_verify): a setup call (allocates, synchronises); results are the same bits
    whatever it picks.  Returns the item size now in use (0: nothing to tune)."""
    lib = library()
    _check(lib.sv_tune_verify(ctypes.byref(model.struct), int(B), int(gamma), _stream(stream)))
    return int(lib.sv_tuned_item(ctypes.byref(model.struct), int(B), int(gamma)))


class Workspace:
    """Caller-owned scratch for the library, grown on demand (one per device).
    Allocated zero-filled, as the library requires of a new workspace (it keeps
    counters and a launch epoch in it between calls).  ``reset()`` zero-fills it
    again (needed only after a sampling step that found part of its grid not
    started; see the header)."""

    def __init__(self):
        self.buf = None

    def reset(self):
        if self.buf is not None:
            self.buf.zero_()

    def get(self, nbytes, device):
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_default_ws = {}


def _workspace(ws, device):
    if ws is not None:
        return ws
    key = device.index
    if key not in _default_ws:
        _default_ws[key] = Workspace()
    return _default_ws[key]


def _call_with_ws(fn, args_before_ws, device, ws, stream):
    """Two-phase call: size query, then the real call."""
    nbytes = ctypes.c_size_t(0)
    _check(fn(*args_before_ws, None, ctypes.byref(nbytes), None))
    buf = _workspace(ws, device).get(nbytes.value, device)
    nbytes = ctypes.c_size_t(buf.numel())
    _check(fn(*args_before_ws, ctypes.c_void_p(buf.data_ptr()), ctypes.byref(nbytes), _stream(stream)))


def _kind_input(kind, inp):
    dt = {SV_IN_LOGITS: torch.float32, SV_IN_TOKENS: torch.int32}.get(kind)
    return _dev_tensor(inp, "input", dt)


def verify_forward(model, kind, inp, B, gamma, kv=None, logits=None, ws=None, stream=None):
    """Logits [B, gamma+1, V] float32 of all slots (C: verify_forward)."""
    lib = library()
    inp = _kind_input(kind, inp)
    if logits is None:
        logits = torch.empty((B, gamma + 1, model.vocab), dtype=torch.float32, device=inp.device)
    _dev_tensor(logits, "logits", torch.float32)
    kvs = kv.struct() if kv is not None else None
    _call_with_ws(lib.verify_forward,
                  (ctypes.byref(model.struct), kind, _ptr(inp), B, gamma,
                   ctypes.byref(kvs) if kvs is not None else None, _ptr(logits)),
                  inp.device, ws, stream)
    return logits


def _outs(B, gamma, device, out):
    if out is not None:
        n, tok = out
        _dev_tensor(n, "n_accepted", torch.int32)
        _dev_tensor(tok, "tokens_out", torch.int32)
        return n, tok
    return (torch.empty(B, dtype=torch.int32, device=device),
            torch.empty((B, gamma + 1), dtype=torch.int32, device=device))


def spec_verify_greedy(model, kind, inp, B, gamma, draft=None, kv=None, logits_out=None, out=None, ws=None,
                       stream=None, diag=None):
    """Greedy verify (C: spec_verify_greedy).  Returns (n_accepted [B], tokens_out [B, gamma+1]).
    ``diag``: optional float32 [B, gamma+1] filled with the per-slot margins."""
    lib = library()
    inp = _kind_input(kind, inp)
    _dev_tensor(draft, "draft", torch.int32)
    _dev_tensor(logits_out, "logits_out", torch.float32)
    _dev_tensor(diag, "diag", torch.float32)
    n, tok = _outs(B, gamma, inp.device, out)
    kvs = kv.struct() if kv is not None else None
    _call_with_ws(lib.spec_verify_greedy,
                  (ctypes.byref(model.struct), kind, _ptr(inp), B, gamma, _ptr(draft),
                   ctypes.byref(kvs) if kvs is not None else None, _ptr(n), _ptr(tok), _ptr(logits_out),
                   _ptr(diag)),
                  inp.device, ws, stream)
    return n, tok


def spec_verify_sample(model, kind, inp, B, gamma, draft, q, temperature, seed, pos0, kv=None, logits_out=None,
                       out=None, ws=None, stream=None, diag=None):
    """Speculative-sampling verify (C: spec_verify_sample).  ``q`` is float32 or
    bfloat16 [B, gamma, V]; ``pos0`` int64 [B].  Returns (n_accepted, tokens_out)."""
    lib = library()
    inp = _kind_input(kind, inp)
    _dev_tensor(draft, "draft", torch.int32)
    _dev_tensor(q, "q")
    _dev_tensor(pos0, "pos0", torch.int64)
    _dev_tensor(logits_out, "logits_out", torch.float32)
    if q.dtype == torch.bfloat16:
        qd = SV_BF16
    elif q.dtype == torch.float32:
        qd = SV_F32
    else:
        raise ValueError("q must be float32 or bfloat16")
    _dev_tensor(diag, "diag", torch.float32)
    n, tok = _outs(B, gamma, inp.device, out)
    kvs = kv.struct() if kv is not None else None
    _call_with_ws(lib.spec_verify_sample,
                  (ctypes.byref(model.struct), kind, _ptr(inp), B, gamma, _ptr(draft), _ptr(q), qd,
                   float(temperature), ctypes.c_uint64(int(seed)), _ptr(pos0),
                   ctypes.byref(kvs) if kvs is not None else None, _ptr(n), _ptr(tok), _ptr(logits_out),
                   _ptr(diag)),
                  inp.device, ws, stream)
    return n, tok


def spec_verify_sample_noalloc(model, kind, inp, B, gamma, draft, q, temperature, seed, pos0, kv=None,
                               logits_out=None, out=None, stream=None, diag=None):
    """spec_verify_sample without a workspace (C: spec_verify_sample_noalloc): the library's
    fixed per-device scratch array serves instead; nothing is allocated by the library.
    Returns (n_accepted, tokens_out); ``out`` may supply them."""
    lib = library()
    inp = _kind_input(kind, inp)
    _dev_tensor(draft, "draft", torch.int32)
    _dev_tensor(q, "q")
    _dev_tensor(pos0, "pos0", torch.int64)
    _dev_tensor(logits_out, "logits_out", torch.float32)
    if q.dtype == torch.bfloat16:
        qd = SV_BF16
    elif q.dtype == torch.float32:
        qd = SV_F32
    else:
        raise ValueError("q must be float32 or bfloat16")
    n, tok = _outs(B, gamma, inp.device, out)
    kvs = kv.struct() if kv is not None else None
    _check(lib.spec_verify_sample_noalloc(ctypes.byref(model.struct), kind, _ptr(inp), B, gamma, _ptr(draft), _ptr(q),
                                          qd, float(temperature), ctypes.c_uint64(int(seed)), _ptr(pos0),
                                          ctypes.byref(kvs) if kvs is not None else None, _ptr(n), _ptr(tok),
                                          _ptr(logits_out), _ptr(diag), _stream(stream)))
    return n, tok


def spec_verify_sample_filtered(model, kind, inp, B, gamma, draft, q, temperature, top_k, top_p, seed, pos0,
                                kv=None, logits_out=None, out=None, ws=None, stream=None):
    """Speculative-sampling verify with the drafter's top-k / top-p filters applied to
    the target alike (C: spec_verify_sample_filtered).  ``q`` is the drafter's filtered
    distributions, float32 or bfloat16 [B, gamma, V]; ``pos0`` int64 [B]; ``top_k`` in
    1..64, ``top_p`` in (0, 1].  Returns (n_accepted, tokens_out)."""
    lib = library()
    inp = _kind_input(kind, inp)
    _dev_tensor(draft, "draft", torch.int32)
    _dev_tensor(q, "q")
    _dev_tensor(pos0, "pos0", torch.int64)
    _dev_tensor(logits_out, "logits_out", torch.float32)
    if q.dtype == torch.bfloat16:
        qd = SV_BF16
    elif q.dtype == torch.float32:
        qd = SV_F32
    else:
        raise ValueError("q must be float32 or bfloat16")
    n, tok = _outs(B, gamma, inp.device, out)
    kvs = kv.struct() if kv is not None else None
    _call_with_ws(lib.spec_verify_sample_filtered,
                  (ctypes.byref(model.struct), kind, _ptr(inp), B, gamma, _ptr(draft), _ptr(q), qd,
                   float(temperature), int(top_k), float(top_p), ctypes.c_uint64(int(seed)), _ptr(pos0),
                   ctypes.byref(kvs) if kvs is not None else None, _ptr(n), _ptr(tok), _ptr(logits_out)),
                  inp.device, ws, stream)
    return n, tok


DRAFTER_LAYER_KEYS = ("attn_norm", "wq", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


@dataclass
class Drafter:
    """The MTP drafter: the C struct plus the tensors and host arrays it points to."""
    struct: _SvDrafter
    keep: list = field(default_factory=list)


def drafter(embed, pre_proj, layers, final_norm, post_proj, n_heads, head_dim, centroids=None, top_k_clusters=0,
            rms_eps=1e-5, rope_theta=10000.0):
    """Drafter from bf16 device tensors: token table [V, D] (shared with the target),
    pre_proj [H, 2D], ``layers`` a list of dicts with DRAFTER_LAYER_KEYS, final_norm [H],
    post_proj [D, H]; ``centroids`` [C, D] selects the centroid-masked head."""
    ts = [embed, pre_proj, final_norm, post_proj] + ([centroids] if centroids is not None else [])
    for t in ts:
        _dev_tensor(t, "drafter weight", torch.bfloat16)
    ptrs = []
    for L in layers:
        for k in DRAFTER_LAYER_KEYS:
            _dev_tensor(L[k], k, torch.bfloat16)
            ptrs.append(L[k].data_ptr())
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    s = _SvDrafter()
    s.n_layers, s.d_model, s.hidden = len(layers), int(embed.shape[1]), int(pre_proj.shape[0])
    s.n_heads, s.head_dim = int(n_heads), int(head_dim)
    s.d_ff, s.vocab = int(layers[0]["w_gate"].shape[0]), int(embed.shape[0])
    s.rms_eps, s.rope_theta = float(rms_eps), float(rope_theta)
    s.embed, s.pre_proj, s.final_norm, s.post_proj = (embed.data_ptr(), pre_proj.data_ptr(), final_norm.data_ptr(),
                                                      post_proj.data_ptr())
    s.layers = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    s.centroids = centroids.data_ptr() if centroids is not None else None
    s.n_clusters = int(centroids.shape[0]) if centroids is not None else 0
    s.top_k_clusters = int(top_k_clusters)
    return Drafter(s, ts + [L[k] for L in layers for k in DRAFTER_LAYER_KEYS] + [arr])


@dataclass
class SharedKV:
    """The drafter's view of the target cache: the C struct plus what it points to."""
    struct: _SvSharedKV
    keep: list = field(default_factory=list)


def shared_kv(k_layers, v_layers, length):
    """The target cache layers the drafter reads: bf16 device tensors [B, heads, max_len,
    head_dim] per drafter layer (may repeat), ``length`` int32 device [B]."""
    for t in list(k_layers) + list(v_layers):
        _dev_tensor(t, "shared cache", torch.bfloat16)
    _dev_tensor(length, "length", torch.int32)
    ka = (ctypes.c_void_p * len(k_layers))(*[t.data_ptr() for t in k_layers])
    va = (ctypes.c_void_p * len(v_layers))(*[t.data_ptr() for t in v_layers])
    s = _SvSharedKV()
    s.k = ctypes.cast(ka, ctypes.POINTER(ctypes.c_void_p))
    s.v = ctypes.cast(va, ctypes.POINTER(ctypes.c_void_p))
    s.max_len = int(k_layers[0].shape[2])
    s.len = length.data_ptr()
    return SharedKV(s, list(k_layers) + list(v_layers) + [length, ka, va])


def mtp_draft(dr, kv, last_token, h_target, gamma, temperature, seed, q_dtype=None, draft=None, q=None, ws=None,
              stream=None):
    """gamma drafter steps (C: mtp_draft).  Returns (draft int32 [B, gamma], q [B, gamma,
    V] or None at T = 0).  ``q_dtype`` torch.float32 (default) or torch.bfloat16."""
    lib = library()
    _dev_tensor(last_token, "last_token", torch.int32)
    _dev_tensor(h_target, "h_target", torch.bfloat16)
    B, dev = int(last_token.shape[0]), last_token.device
    V = dr.struct.vocab
    if draft is None:
        draft = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    _dev_tensor(draft, "draft", torch.int32)
    qd = SV_F32
    if float(temperature) > 0.0:
        dt = q_dtype or (q.dtype if q is not None else torch.float32)
        if q is None:
            q = torch.empty((B, gamma, V), dtype=dt, device=dev)
        _dev_tensor(q, "q", dt)
        qd = SV_BF16 if dt == torch.bfloat16 else SV_F32
    _call_with_ws(lib.mtp_draft,
                  (ctypes.byref(dr.struct), ctypes.byref(kv.struct), B, int(gamma), _ptr(last_token), _ptr(h_target),
                   float(temperature), ctypes.c_uint64(int(seed)), _ptr(draft), _ptr(q), qd),
                  dev, ws, stream)
    return draft, q


def round_pad_drafts(gamma_b, draft, q=None, tau=0.0, ws=None, stream=None):
    """Per-sequence draft length by padding (C: round_pad_drafts): ``gamma_b`` int32 [B]
    (updated in place: clamped, and cut by the confidence rule when tau > 0), ``draft``
    int32 [B, G] and ``q`` [B, G, V] (float32 or bfloat16, or None) padded in place."""
    lib = library()
    _dev_tensor(gamma_b, "gamma_b", torch.int32)
    _dev_tensor(draft, "draft", torch.int32)
    _dev_tensor(q, "q")
    B, G = int(draft.shape[0]), int(draft.shape[1])
    V = int(q.shape[2]) if q is not None else 1
    qd = SV_BF16 if (q is not None and q.dtype == torch.bfloat16) else SV_F32
    _call_with_ws(lib.round_pad_drafts, (B, G, V, _ptr(gamma_b), _ptr(draft), _ptr(q), qd, float(tau)),
                  draft.device, ws, stream)


def round_update_gamma(n_accepted, gamma_b, gamma_min=1, gamma_max=15, stream=None):
    """Heuristic schedule in place on ``gamma_b`` (C: round_update_gamma)."""
    _dev_tensor(n_accepted, "n_accepted", torch.int32)
    _dev_tensor(gamma_b, "gamma_b", torch.int32)
    _check(library().round_update_gamma(int(gamma_b.shape[0]), _ptr(n_accepted), _ptr(gamma_b), int(gamma_min),
                                        int(gamma_max), _stream(stream)))


def round_select_candidates(n_accepted, tokens, stream=None):
    """The longest accepted of C candidates per sequence (C: round_select_candidates):
    ``n_accepted`` int32 [B, C], ``tokens`` int32 [B, C, G1].  Returns (best [B],
    n [B], tokens [B, G1])."""
    _dev_tensor(n_accepted, "n_accepted", torch.int32)
    _dev_tensor(tokens, "tokens", torch.int32)
    B, C, G1 = (int(x) for x in tokens.shape)
    dev = tokens.device
    best = torch.empty(B, dtype=torch.int32, device=dev)
    n = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty((B, G1), dtype=torch.int32, device=dev)
    _check(library().round_select_candidates(B, C, G1, _ptr(n_accepted), _ptr(tokens), _ptr(best), _ptr(n),
                                             _ptr(tok), _stream(stream)))
    return best, n, tok


def timing_enable(mask=0b111):
    """Start event timing of the kernel classes in ``mask`` (bit 0 LM-head
    product, bit 1 decoder layers, bit 2 acceptance tail), clearing earlier
    records; ``mask=0`` stops."""
    _check(library().sv_timing_enable(int(mask)))


def timing_read(which):
    """(total milliseconds, launches) recorded for class ``which``
    (0 LM-head product, 1 decoder layers, 2 acceptance tail)."""
    ms, cnt = ctypes.c_double(0), ctypes.c_int64(0)
    _check(library().sv_timing_read(which, ctypes.byref(ms), ctypes.byref(cnt)))
    return ms.value, cnt.value


@dataclass
class MaskedHead:
    """The drafter's centroid-masked LM head: the C struct plus the tensors it points to."""
    struct: _SvMaskedHead
    keep: list = field(default_factory=list)

    @property
    def cluster_size(self):
        return self.struct.vocab // self.struct.n_clusters


def masked_head(embed, centroids):
    """Masked head from bf16 device tensors: cluster-ordered token table [V, d] and one
    representative embedding per cluster [C, d] (cluster c = tokens [c*V/C, (c+1)*V/C))."""
    _dev_tensor(embed, "embed", torch.bfloat16)
    _dev_tensor(centroids, "centroids", torch.bfloat16)
    s = _SvMaskedHead()
    s.vocab, s.d_model = int(embed.shape[0]), int(embed.shape[1])
    s.n_clusters = int(centroids.shape[0])
    s.wdtype = SV_BF16
    s.embed, s.centroids = embed.data_ptr(), centroids.data_ptr()
    return MaskedHead(s, [embed, centroids])


def draft_masked_logits(head, hidden, top_k, clusters=None, logits=None, cluster_logits=None, ws=None, stream=None):
    """(clusters int32 [M, top_k], logits float32 [M, top_k * cs]) of the masked head
    (C: draft_masked_logits); ``hidden`` bf16 [M, d]."""
    lib = library()
    _dev_tensor(hidden, "hidden", torch.bfloat16)
    M, dev = int(hidden.shape[0]), hidden.device
    if clusters is None:
        clusters = torch.empty((M, top_k), dtype=torch.int32, device=dev)
    if logits is None:
        logits = torch.empty((M, top_k * head.cluster_size), dtype=torch.float32, device=dev)
    _dev_tensor(clusters, "clusters", torch.int32)
    _dev_tensor(logits, "logits", torch.float32)
    _dev_tensor(cluster_logits, "cluster_logits", torch.float32)
    st = head.struct
    _call_with_ws(lib.draft_masked_logits,
                  (ctypes.byref(st), _ptr(hidden), M, int(top_k), _ptr(clusters), _ptr(logits), _ptr(cluster_logits)),
                  dev, ws, stream)
    return clusters, logits
