"""fp64 CPU oracle for batched speculative-sampling verification, VAT labels and
the VAT training loss.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
bench's CPU-baseline leg are its only callers.  The product path never imports
this package, and this package imports nothing from the product path.

The arithmetic lives in ``oracle.c`` (plain C, fp64, one row at a time); this
module only marshals numpy arrays into it through ctypes.  The sources each
function follows are cited in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.environ.get("ORACLE_LIB_OVERRIDE") or os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
F64 = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-fPIC", "-shared", "-fno-fast-math",
             "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    c = ctypes
    vp = c.c_void_p
    lib.orc_abi_version.restype = c.c_int
    lib.orc_decode_bf16.argtypes = [c.c_uint16]
    lib.orc_decode_bf16.restype = c.c_double
    lib.orc_decode_f32.argtypes = [c.c_uint32]
    lib.orc_decode_f32.restype = c.c_double
    lib.orc_softmax.argtypes = [vp, c.c_int64, c.c_double, vp, vp, vp]
    lib.orc_softmax.restype = None
    lib.orc_argmax.argtypes = [vp, c.c_int64]
    lib.orc_argmax.restype = c.c_int64
    lib.orc_accept_prob.argtypes = [c.c_double, c.c_double]
    lib.orc_accept_prob.restype = c.c_double
    lib.orc_accept.argtypes = [c.c_double, c.c_double, c.c_double]
    lib.orc_accept.restype = c.c_int
    lib.orc_residual.argtypes = [vp, vp, c.c_int64, vp]
    lib.orc_residual.restype = None
    lib.orc_inverse_cdf.argtypes = [vp, c.c_int64, c.c_double, vp]
    lib.orc_inverse_cdf.restype = c.c_int64
    lib.orc_verify.argtypes = [c.c_int64, c.c_int32, c.c_int64, c.c_int32, c.c_int32, c.c_double,
                               vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_verify.restype = c.c_int
    lib.orc_vat.argtypes = [c.c_int64, c.c_int32, c.c_int64, c.c_int32, c.c_double, c.c_double,
                            vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_vat.restype = c.c_int
    lib.orc_vat_loss.argtypes = [c.c_int64, c.c_int32, c.c_int64, c.c_int32, c.c_double, c.c_double, c.c_double,
                                 vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_vat_loss.restype = c.c_int
    lib.orc_vat_loss_grad.argtypes = [c.c_int64, c.c_int32, c.c_int64, c.c_int32, c.c_double, c.c_double,
                                      vp, vp, vp, vp, vp]
    lib.orc_vat_loss_grad.restype = c.c_int
    lib.orc_lm_head_greedy.argtypes = [c.c_int64, c.c_int32, c.c_int64, c.c_int64, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_lm_head_greedy.restype = c.c_int
    lib.orc_lm_head_logits.argtypes = [c.c_int64, c.c_int64, c.c_int64, vp, vp, vp]
    lib.orc_lm_head_logits.restype = c.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logits_arg(a):
    """Logits arrive as float32, or as uint16 holding bfloat16 bit patterns."""
    if a is None:
        return None, None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.float64:
        return a, F64
    raise TypeError("logits must be float32, float64 or uint16 (bfloat16 bits), got %s" % a.dtype)


# ---------------------------------------------------------------- primitives

def decode_bf16(bits) -> np.ndarray:
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_decode_bf16(int(b)) for b in bits], dtype=np.float64)


def softmax(logits, T: float):
    """Returns (p, m, Z) for one row of fp64 logits at temperature T > 0."""
    lib = _load()
    l = np.ascontiguousarray(logits, dtype=np.float64)
    p = np.empty_like(l)
    m = ctypes.c_double()
    z = ctypes.c_double()
    lib.orc_softmax(_ptr(l), l.size, float(T), _ptr(p), ctypes.byref(m), ctypes.byref(z))
    return p, m.value, z.value


def argmax(logits) -> int:
    lib = _load()
    l = np.ascontiguousarray(logits, dtype=np.float64)
    return int(lib.orc_argmax(_ptr(l), l.size))


def accept_prob(p: float, q: float) -> float:
    return float(_load().orc_accept_prob(float(p), float(q)))


def accept(u: float, p: float, q: float) -> bool:
    return bool(_load().orc_accept(float(u), float(p), float(q)))


def residual(p, q) -> np.ndarray:
    lib = _load()
    p = np.ascontiguousarray(p, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    assert p.shape == q.shape
    w = np.empty_like(p)
    lib.orc_residual(_ptr(p), _ptr(q), p.size, _ptr(w))
    return w


def inverse_cdf(w, u: float):
    """Returns (index, margin)."""
    lib = _load()
    w = np.ascontiguousarray(w, dtype=np.float64)
    margin = ctypes.c_double()
    y = lib.orc_inverse_cdf(_ptr(w), w.size, float(u), ctypes.byref(margin))
    return int(y), margin.value


# ---------------------------------------------------------------- batched paths

class VerifyResult:
    __slots__ = ("accepted_len", "out_tokens", "probs", "target_mz", "draft_mz",
                 "accept_margin", "sample_margin")

    def __init__(self, **kw):
        for k, v in kw.items():
            setattr(self, k, v)


def verify(target, draft, tokens, uniforms, temperature: float, onehot: bool = False) -> VerifyResult:
    """Batched verification.

    target: [B][k+1][V] float32 or uint16 (bf16 bits); draft: [B][k][V] same dtype
    (None if onehot or temperature == 0); tokens: [B][k] int32; uniforms: [B][k+1]
    float32 (None allowed at temperature 0).
    """
    lib = _load()
    t, dt = _logits_arg(target)
    B, kp1, V = t.shape
    k = kp1 - 1
    d = None
    if draft is not None and not onehot and temperature != 0.0:
        d, dd = _logits_arg(draft)
        assert dd == dt and d.shape == (B, k, V)
    x = np.ascontiguousarray(tokens, dtype=np.int32)
    assert x.shape == (B, k)
    u = None if uniforms is None else np.ascontiguousarray(uniforms, dtype=np.float32)
    if u is not None:
        assert u.shape == (B, k + 1)
    acc = np.empty(B, np.int32)
    out = np.empty((B, k + 1), np.int32)
    probs = np.empty((B, k, 2), np.float64)
    tmz = np.empty((B, k + 1, 2), np.float64)
    dmz = np.empty((B, k, 2), np.float64)
    am = np.empty((B, k), np.float64)
    sm = np.empty(B, np.float64)
    rc = lib.orc_verify(B, k, V, dt, int(bool(onehot)), float(temperature), _ptr(t), _ptr(d),
                        _ptr(x), _ptr(u), _ptr(acc), _ptr(out), _ptr(probs), _ptr(tmz), _ptr(dmz),
                        _ptr(am), _ptr(sm))
    if rc != 0:
        raise ValueError("orc_verify rejected its arguments")
    return VerifyResult(accepted_len=acc, out_tokens=out, probs=probs, target_mz=tmz,
                        draft_mz=dmz, accept_margin=am, sample_margin=sm)


class VatResult:
    __slots__ = ("accept_mask", "first_reject", "weights", "probs", "target_mz", "draft_mz",
                 "accept_margin", "soft", "hard", "block_loss")

    def __init__(self, **kw):
        for k, v in kw.items():
            setattr(self, k, v)


def vat_labels(target, draft, tokens, uniforms, temperature: float, decay: float) -> VatResult:
    """VAT labels. target/draft: [N][k][V]; tokens, uniforms: [N][k]."""
    lib = _load()
    t, dt = _logits_arg(target)
    N, k, V = t.shape
    d = None
    if temperature != 0.0:
        d, dd = _logits_arg(draft)
        assert dd == dt and d.shape == (N, k, V)
    x = np.ascontiguousarray(tokens, dtype=np.int32)
    assert x.shape == (N, k)
    u = None if uniforms is None else np.ascontiguousarray(uniforms, dtype=np.float32)
    mask = np.empty((N, k), np.uint8)
    fr = np.empty(N, np.int32)
    w = np.empty((N, k), np.float64)
    probs = np.empty((N, k, 2), np.float64)
    tmz = np.empty((N, k, 2), np.float64)
    dmz = np.empty((N, k, 2), np.float64)
    am = np.empty((N, k), np.float64)
    rc = lib.orc_vat(N, k, V, dt, float(temperature), float(decay), _ptr(t), _ptr(d), _ptr(x),
                     _ptr(u), _ptr(mask), _ptr(fr), _ptr(w), _ptr(probs), _ptr(tmz), _ptr(dmz),
                     _ptr(am))
    if rc != 0:
        raise ValueError("orc_vat rejected its arguments")
    return VatResult(accept_mask=mask, first_reject=fr, weights=w, probs=probs, target_mz=tmz,
                     draft_mz=dmz, accept_margin=am)


def vat_loss(target, draft, tokens, uniforms, hard_tokens, temperature: float, decay: float,
             hard_weight: float = 1.0) -> VatResult:
    """VAT labels plus the weighted training loss of each block: soft term
    -sum p ln q, hard term -ln q(h), block loss sum_i w_i (soft_i +
    hard_weight * hard_i).  target/draft: [N][k][V]; tokens, uniforms,
    hard_tokens: [N][k]; temperature > 0."""
    lib = _load()
    t, dt = _logits_arg(target)
    N, k, V = t.shape
    d, dd = _logits_arg(draft)
    assert dd == dt and d.shape == (N, k, V)
    x = np.ascontiguousarray(tokens, dtype=np.int32)
    h = np.ascontiguousarray(hard_tokens, dtype=np.int32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    assert x.shape == (N, k) and h.shape == (N, k) and u.shape == (N, k)
    mask = np.empty((N, k), np.uint8)
    fr = np.empty(N, np.int32)
    w = np.empty((N, k), np.float64)
    soft = np.empty((N, k), np.float64)
    hard = np.empty((N, k), np.float64)
    loss = np.empty(N, np.float64)
    rc = lib.orc_vat_loss(N, k, V, dt, float(temperature), float(decay), float(hard_weight), _ptr(t), _ptr(d),
                          _ptr(x), _ptr(u), _ptr(h), _ptr(mask), _ptr(fr), _ptr(w), _ptr(soft), _ptr(hard),
                          _ptr(loss))
    if rc != 0:
        raise ValueError("orc_vat_loss rejected its arguments")
    return VatResult(accept_mask=mask, first_reject=fr, weights=w, soft=soft, hard=hard, block_loss=loss)


def vat_loss_grad(target, draft, hard_tokens, weights, temperature: float, hard_weight: float = 1.0) -> np.ndarray:
    """d(block loss)/d(draft logits), [N][k][V] fp64, with the weights (as
    returned by vat_loss) held fixed: w_i/T ((1 + hard_weight) q - p - hard_weight e_h)."""
    lib = _load()
    t, dt = _logits_arg(target)
    N, k, V = t.shape
    d, dd = _logits_arg(draft)
    assert dd == dt and d.shape == (N, k, V)
    h = np.ascontiguousarray(hard_tokens, dtype=np.int32)
    w = np.ascontiguousarray(weights, dtype=np.float64)
    assert h.shape == (N, k) and w.shape == (N, k)
    g = np.empty((N, k, V), np.float64)
    rc = lib.orc_vat_loss_grad(N, k, V, dt, float(temperature), float(hard_weight), _ptr(t), _ptr(d), _ptr(h),
                               _ptr(w), _ptr(g))
    if rc != 0:
        raise ValueError("orc_vat_loss_grad rejected its arguments")
    return g


class LmHeadResult:
    __slots__ = ("accepted_len", "out_tokens", "argmax", "top2_gap")

    def __init__(self, **kw):
        for k, v in kw.items():
            setattr(self, k, v)


def lm_head_greedy(hidden, weight, tokens) -> LmHeadResult:
    """Greedy verification with logits formed from hidden states: hidden
    [B][k+1][D] and weight [V][D] as bf16 bit patterns (uint16), tokens
    [B][k].  fp64 logits, lowest-index argmax."""
    lib = _load()
    h = np.ascontiguousarray(hidden, dtype=np.uint16)
    w = np.ascontiguousarray(weight, dtype=np.uint16)
    B, kp1, D = h.shape
    V, D2 = w.shape
    assert D2 == D
    k = kp1 - 1
    x = np.ascontiguousarray(tokens, dtype=np.int32)
    assert x.shape == (B, k)
    acc = np.empty(B, np.int32)
    out = np.empty((B, k + 1), np.int32)
    am = np.empty((B, k + 1), np.int32)
    gap = np.empty((B, k + 1), np.float64)
    rc = lib.orc_lm_head_greedy(B, k, V, D, _ptr(h), _ptr(w), _ptr(x), _ptr(acc), _ptr(out), _ptr(am), _ptr(gap))
    if rc != 0:
        raise ValueError("orc_lm_head_greedy rejected its arguments")
    return LmHeadResult(accepted_len=acc, out_tokens=out, argmax=am, top2_gap=gap)


def lm_head_logits(hidden, weight) -> np.ndarray:
    """fp64 logits hidden . weight^T from bf16 bit patterns: hidden [..., D],
    weight [V][D]; returns [..., V] float64."""
    lib = _load()
    h = np.ascontiguousarray(hidden, dtype=np.uint16)
    w = np.ascontiguousarray(weight, dtype=np.uint16)
    V, D = w.shape
    assert h.shape[-1] == D
    rows = int(np.prod(h.shape[:-1]))
    out = np.empty(h.shape[:-1] + (V,), np.float64)
    rc = lib.orc_lm_head_logits(rows, V, D, _ptr(h), _ptr(w), _ptr(out))
    if rc != 0:
        raise ValueError("orc_lm_head_logits rejected its arguments")
    return out


def lm_head_verify(target_hidden, target_weight, draft_hidden, draft_weight, tokens, uniforms,
                   temperature: float) -> VerifyResult:
    """Verification at T > 0 with both distributions formed from hidden
    states: p = softmax(H_t W_t^T / T), q = softmax(H_d W_d^T / T) in fp64, then
    the rule of verify()."""
    assert temperature > 0.0
    lt = lm_head_logits(target_hidden, target_weight)
    ld = lm_head_logits(draft_hidden, draft_weight)
    return verify(lt, ld, tokens, uniforms, temperature)
