"""Python binding of libspecverify (batched speculative-sampling verification on MI355X).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and the stream (the current
torch stream of the tensors' device).  There is no CPU fallback: if the
library is not built, importing works but every call raises.

    from speculative_decoding_verification_amd import verify, vat_labels
    acc, out = verify(target, draft, tokens, uniforms, temperature=1.0)

Names follow the C ABI in ``include/specverify.h``: ``sv_verify`` (and
``sv_verify_ex`` when row statistics or a probe are asked for) ->
:func:`verify`, ``sv_vat_labels`` (``sv_vat_labels_ex``) -> :func:`vat_labels`, ``sv_vat_loss`` ->
:func:`vat_loss`, ``sv_verify_lm_head_greedy`` -> :func:`verify_lm_head_greedy`,
``sv_verify_lm_head`` -> :func:`verify_lm_head`.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

__all__ = ["verify", "verify_noalloc", "vat_labels", "vat_loss", "verify_lm_head_greedy", "verify_lm_head", "accept_histogram",
           "Verifier", "VatLabeler", "VatLoss", "LmHeadVerifier", "LmHeadSampler",
           "DraftLengthController", "SVError", "library_path", "load_library", "SV_F32", "SV_BF16", "SV_DRAFT_LOGITS",
           "SV_DRAFT_ONEHOT", "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
SV_DRAFT_LOGITS, SV_DRAFT_ONEHOT = 0, 1
STATUS = {0: "SV_OK", 1: "SV_ERR_NULL_ARG", 2: "SV_ERR_BAD_SHAPE", 3: "SV_ERR_BAD_DTYPE",
          4: "SV_ERR_BAD_TEMPERATURE", 5: "SV_ERR_WORKSPACE_TOO_SMALL", 6: "SV_ERR_HIP",
          7: "SV_ERR_BAD_DRAFT_KIND", 8: "SV_ERR_BAD_DECAY", 9: "SV_ERR_BAD_HARD_WEIGHT", 10: "SV_ERR_BAD_CONTROL",
          11: "SV_ERR_MISALIGNED", 12: "SV_ERR_CAPTURING", 13: "SV_ERR_SCRATCH_TOO_SMALL"}
STATUS_CODE = {name: code for code, name in STATUS.items()}

EXPORTED_SYMBOLS = ("sv_abi_version", "sv_status_str", "sv_verify_workspace_bytes", "sv_verify", "sv_verify_ex",
                    "sv_verify_noalloc",
                    "sv_vat_workspace_bytes", "sv_vat_labels", "sv_vat_labels_ex", "sv_vat_loss_workspace_bytes",
                    "sv_vat_loss", "sv_vat_loss_grad",
                    "sv_lm_head_workspace_bytes", "sv_verify_lm_head_greedy", "sv_lm_head_sample_workspace_bytes",
                    "sv_verify_lm_head", "sv_accept_histogram",
                    "sv_draft_len_init", "sv_draft_len_update", "sv_sol_read", "sv_sol_read_write")


class SVError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        self.status = status
        msg = STATUS.get(status, "status %d" % status)
        if lib is not None and hasattr(lib, "sv_status_str"):
            lib.sv_status_str.restype = ctypes.c_char_p
            msg = lib.sv_status_str(status).decode()
        super().__init__("%s: %s" % (where, msg))


class VerifyDesc(ctypes.Structure):
    """sv_verify_desc: B, k, V, dtype (sv_dtype), draft_kind (sv_draft_kind), temperature."""
    _fields_ = [("B", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("draft_kind", ctypes.c_int32), ("temperature", ctypes.c_float)]


class VatDesc(ctypes.Structure):
    """sv_vat_desc: N, k, V, dtype, temperature, decay."""
    _fields_ = [("N", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("temperature", ctypes.c_float), ("decay", ctypes.c_float)]


class VatLossDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("temperature", ctypes.c_float), ("decay", ctypes.c_float),
                ("hard_weight", ctypes.c_float)]


class LmHeadDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32), ("D", ctypes.c_int32)]


class LmHeadSampleDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32), ("D", ctypes.c_int32),
                ("temperature", ctypes.c_float)]


class Probe(ctypes.Structure):
    """sv_probe: two hipEvent_t handles recorded around a call's main kernel."""
    _fields_ = [("start", ctypes.c_void_p), ("stop", ctypes.c_void_p)]


SV_MAX_DRAFT_CHOICES = 8


class DraftLenCtl(ctypes.Structure):
    _fields_ = [("n_choices", ctypes.c_int32), ("choices", ctypes.c_int32 * SV_MAX_DRAFT_CHOICES),
                ("index", ctypes.c_int32), ("up_frac", ctypes.c_float), ("down_frac", ctypes.c_float),
                ("patience", ctypes.c_int32), ("up_streak", ctypes.c_int32), ("down_streak", ctypes.c_int32),
                ("last_efficiency", ctypes.c_float)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Loads libspecverify.so (built in-tree).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libspecverify.so is not built (%s); run "
                           "`python -m speculative_decoding_verification_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.sv_abi_version.restype = ctypes.c_int
    lib.sv_abi_version.argtypes = []
    lib.sv_status_str.restype = ctypes.c_char_p
    lib.sv_status_str.argtypes = [ctypes.c_int]
    pr = ctypes.POINTER(Probe)
    lib.sv_verify_workspace_bytes.restype = sz
    lib.sv_verify_workspace_bytes.argtypes = [ctypes.POINTER(VerifyDesc)]
    lib.sv_verify.restype = ctypes.c_int
    lib.sv_verify.argtypes = [ctypes.POINTER(VerifyDesc)] + [vp] * 8 + [sz, vp]
    lib.sv_verify_ex.restype = ctypes.c_int
    lib.sv_verify_ex.argtypes = [ctypes.POINTER(VerifyDesc)] + [vp] * 8 + [pr, vp, sz, vp]
    lib.sv_verify_noalloc.restype = ctypes.c_int
    lib.sv_verify_noalloc.argtypes = [ctypes.POINTER(VerifyDesc)] + [vp] * 8
    lib.sv_vat_workspace_bytes.restype = sz
    lib.sv_vat_workspace_bytes.argtypes = [ctypes.POINTER(VatDesc)]
    lib.sv_vat_labels.restype = ctypes.c_int
    lib.sv_vat_labels.argtypes = [ctypes.POINTER(VatDesc)] + [vp] * 9 + [sz, vp]
    lib.sv_vat_labels_ex.restype = ctypes.c_int
    lib.sv_vat_labels_ex.argtypes = [ctypes.POINTER(VatDesc)] + [vp] * 9 + [pr, vp, sz, vp]
    lib.sv_vat_loss_workspace_bytes.restype = sz
    lib.sv_vat_loss_workspace_bytes.argtypes = [ctypes.POINTER(VatLossDesc)]
    lib.sv_vat_loss.restype = ctypes.c_int
    lib.sv_vat_loss.argtypes = [ctypes.POINTER(VatLossDesc)] + [vp] * 13 + [pr, vp, sz, vp]
    lib.sv_vat_loss_grad.restype = ctypes.c_int
    lib.sv_vat_loss_grad.argtypes = [ctypes.POINTER(VatLossDesc)] + [vp] * 6 + [pr, vp]
    lib.sv_lm_head_workspace_bytes.restype = sz
    lib.sv_lm_head_workspace_bytes.argtypes = [ctypes.POINTER(LmHeadDesc)]
    lib.sv_verify_lm_head_greedy.restype = ctypes.c_int
    lib.sv_verify_lm_head_greedy.argtypes = [ctypes.POINTER(LmHeadDesc)] + [vp] * 6 + [pr, vp, sz, vp]
    lib.sv_lm_head_sample_workspace_bytes.restype = sz
    lib.sv_lm_head_sample_workspace_bytes.argtypes = [ctypes.POINTER(LmHeadSampleDesc)]
    lib.sv_verify_lm_head.restype = ctypes.c_int
    lib.sv_verify_lm_head.argtypes = [ctypes.POINTER(LmHeadSampleDesc)] + [vp] * 9 + [pr, vp, sz, vp]
    i32 = ctypes.c_int32
    lib.sv_accept_histogram.restype = ctypes.c_int
    lib.sv_accept_histogram.argtypes = [vp, i32, i32, vp, vp]
    _bind_control(lib)
    lib.sv_sol_read.restype = ctypes.c_int
    lib.sv_sol_read.argtypes = [vp, sz, vp, vp]
    lib.sv_sol_read_write.restype = ctypes.c_int
    lib.sv_sol_read_write.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int, vp]
    _lib = lib
    return lib


def _bind_control(lib) -> None:
    i32 = ctypes.c_int32
    lib.sv_draft_len_init.restype = ctypes.c_int
    lib.sv_draft_len_init.argtypes = [ctypes.POINTER(DraftLenCtl), ctypes.POINTER(i32), i32, ctypes.c_float,
                                      ctypes.c_float, i32]
    lib.sv_draft_len_update.restype = ctypes.c_int
    lib.sv_draft_len_update.argtypes = [ctypes.POINTER(DraftLenCtl), ctypes.POINTER(i32), i32, ctypes.POINTER(i32)]


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError("logits must be torch.float32 or torch.bfloat16, got %s" % t.dtype)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_dev(name, t, device, dtype=None, shape=None):
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _probe_ref(probe):
    """(start, stop) hipEvent_t handles -> a Probe record (kept by the caller), or None."""
    if probe is None:
        return None
    return Probe(*probe)


def _workspace_bytes(lib, query, call, desc, n_args, name) -> int:
    """Size query; an invalid descriptor (size 0) raises with the reason the
    compute entry point gives for it (it checks the descriptor first)."""
    n = query(ctypes.byref(desc))
    if n == 0:
        st = call(ctypes.byref(desc), *n_args)
        raise SVError(st if st else 2, name, lib)
    return n


class _Workspace:
    """Zero-filled workspaces, one per (device, stream), grown on demand (the
    library allocates nothing).  Calls on one stream run in order and may share
    a workspace; calls on different streams may overlap, so each stream gets
    its own.  The stream is the device's current stream when the call object
    is built: an object built on one stream and called on another needs a
    workspace of its own (the `workspace` argument)."""

    def __init__(self):
        self._buf = {}

    def get(self, device, nbytes: int):
        torch = _torch()
        key = (device, _stream_handle(device))
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._buf[key] = buf
        return buf


# sv_verify / sv_vat_labels / sv_vat_loss hand values between blocks through
# tagged words and need a workspace that only they have written since it was
# zero-filled; the LM-head entry points write plain data and get their own.
_WS = _Workspace()
_WS_LM = _Workspace()


def _stream_handle(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


class VerifyOutput(NamedTuple):
    accepted_len: "object"
    out_tokens: "object"
    probs: "object"
    row_stats: "object"


class Verifier:
    """A prepared sv_verify call: descriptor, outputs and workspace built once,
    so that repeated calls (bench loops, decode steps) only cross ctypes."""

    def __init__(self, target, draft, draft_tokens, uniforms, temperature: float, *, onehot: bool = False,
                 return_probs: bool = False, return_row_stats: bool = False, workspace=None, probe=None):
        torch = _torch()
        lib = load_library()
        if target.dim() != 3:
            raise ValueError("target must be [B][k+1][V]")
        B, kp1, V = (int(s) for s in target.shape)
        k = kp1 - 1
        device = target.device
        dt = _dtype_code(target)
        _check_dev("target", target, device)
        greedy = float(temperature) == 0.0
        uses_draft = (not onehot) and not greedy
        if uses_draft:
            if draft is None:
                raise ValueError("draft logits are required unless onehot or temperature == 0")
            _check_dev("draft", draft, device, target.dtype, (B, k, V))
        else:
            draft = None
        _check_dev("draft_tokens", draft_tokens, device, torch.int32, (B, k))
        if not greedy:
            if uniforms is None:
                raise ValueError("uniforms are required unless temperature == 0")
            _check_dev("uniforms", uniforms, device, torch.float32, (B, k + 1))
        else:
            uniforms = None
        self.desc = VerifyDesc(B, k, V, dt, SV_DRAFT_ONEHOT if onehot else SV_DRAFT_LOGITS, float(temperature))
        nbytes = _workspace_bytes(lib, lib.sv_verify_workspace_bytes, lib.sv_verify, self.desc,
                                  [None] * 8 + [0, None], "sv_verify")
        if workspace is None:
            workspace = _WS.get(device, nbytes)
        elif workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: need %d bytes" % nbytes)
        self.accepted_len = torch.empty(B, dtype=torch.int32, device=device)
        self.out_tokens = torch.empty((B, k + 1), dtype=torch.int32, device=device)
        self.probs = torch.empty((B, k, 2), dtype=torch.float32, device=device) if return_probs else None
        rows = B * (k + 1) + (B * k if uses_draft else 0)
        self.row_stats = torch.empty((rows, 2), dtype=torch.float32, device=device) if return_row_stats else None
        self._keep = (target, draft, draft_tokens, uniforms, workspace)
        self._lib = lib
        self._device = device
        self._head = (ctypes.byref(self.desc), _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                      _ptr(self.accepted_len), _ptr(self.out_tokens), _ptr(self.probs))
        self._ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
        self.set_probe(probe)

    def set_probe(self, probe) -> None:
        """(start, stop) hipEvent_t handles to record around the kernel, or None."""
        self.probe = _probe_ref(probe)

    def __call__(self, stream: Optional[int] = None) -> VerifyOutput:
        s = _stream_handle(self._device) if stream is None else stream
        if self.row_stats is None and self.probe is None:
            st = self._lib.sv_verify(*self._head, *self._ws, s)
            name = "sv_verify"
        else:
            st = self._lib.sv_verify_ex(*self._head, _ptr(self.row_stats),
                                        None if self.probe is None else ctypes.byref(self.probe), *self._ws, s)
            name = "sv_verify_ex"
        if st:
            raise SVError(st, name, self._lib)
        return VerifyOutput(self.accepted_len, self.out_tokens, self.probs, self.row_stats)


def verify(target, draft, draft_tokens, uniforms, temperature: float, *, onehot: bool = False,
           return_probs: bool = False, return_row_stats: bool = False, workspace=None) -> VerifyOutput:
    """sv_verify on torch tensors (all on one HIP device, contiguous).

    target [B][k+1][V] bf16/fp32; draft [B][k][V] same dtype (ignored when
    onehot or temperature == 0); draft_tokens [B][k] int32; uniforms [B][k+1]
    float32 (ignored at temperature 0).  Returns (accepted_len [B],
    out_tokens [B][k+1], probs [B][k][2] or None, row_stats or None).
    Runs on the device's current stream; without `workspace`, each stream
    gets a zero-filled workspace of its own.
    """
    return Verifier(target, draft, draft_tokens, uniforms, temperature, onehot=onehot, return_probs=return_probs,
                    return_row_stats=return_row_stats, workspace=workspace)()


def verify_noalloc(target, draft, draft_tokens, uniforms, temperature: float, *, onehot: bool = False,
                   return_probs: bool = False, stream: Optional[int] = None) -> VerifyOutput:
    """sv_verify_noalloc on torch tensors: as :func:`verify`, with the
    library's built-in per-device workspace instead of one passed in (the
    call itself allocates nothing on the device; the output tensors are
    allocated here).  Calls that overlap on one device must not be issued."""
    torch = _torch()
    lib = load_library()
    B, kp1, V = (int(s) for s in target.shape)
    k = kp1 - 1
    device = target.device
    greedy = float(temperature) == 0.0
    uses_draft = (not onehot) and not greedy
    _check_dev("target", target, device)
    if uses_draft:
        _check_dev("draft", draft, device, target.dtype, (B, k, V))
    _check_dev("draft_tokens", draft_tokens, device, torch.int32, (B, k))
    if not greedy:
        _check_dev("uniforms", uniforms, device, torch.float32, (B, k + 1))
    desc = VerifyDesc(B, k, V, _dtype_code(target), SV_DRAFT_ONEHOT if onehot else SV_DRAFT_LOGITS,
                      float(temperature))
    acc = torch.empty(B, dtype=torch.int32, device=device)
    out = torch.empty((B, k + 1), dtype=torch.int32, device=device)
    probs = torch.empty((B, k, 2), dtype=torch.float32, device=device) if return_probs else None
    s = _stream_handle(device) if stream is None else stream
    st = lib.sv_verify_noalloc(ctypes.byref(desc), _ptr(target), _ptr(draft) if uses_draft else None,
                               _ptr(draft_tokens), _ptr(uniforms) if not greedy else None, _ptr(acc), _ptr(out),
                               _ptr(probs), s)
    if st:
        raise SVError(st, "sv_verify_noalloc", lib)
    return VerifyOutput(acc, out, probs, None)


class VatOutput(NamedTuple):
    accept_mask: "object"
    first_reject: "object"
    weights: "object"
    probs: "object"
    row_stats: "object"


class VatLabeler:
    """A prepared sv_vat_labels call (see :class:`Verifier`)."""

    def __init__(self, target, draft, draft_tokens, uniforms, temperature: float, decay: float, *,
                 return_probs: bool = False, return_row_stats: bool = False, workspace=None, probe=None):
        torch = _torch()
        lib = load_library()
        if target.dim() != 3:
            raise ValueError("target must be [N][k][V]")
        N, k, V = (int(s) for s in target.shape)
        device = target.device
        dt = _dtype_code(target)
        _check_dev("target", target, device)
        greedy = float(temperature) == 0.0
        if not greedy:
            if draft is None or uniforms is None:
                raise ValueError("draft logits and uniforms are required unless temperature == 0")
            _check_dev("draft", draft, device, target.dtype, (N, k, V))
            _check_dev("uniforms", uniforms, device, torch.float32, (N, k))
        else:
            draft, uniforms = None, None
        _check_dev("draft_tokens", draft_tokens, device, torch.int32, (N, k))
        self.desc = VatDesc(N, k, V, dt, float(temperature), float(decay))
        nbytes = _workspace_bytes(lib, lib.sv_vat_workspace_bytes, lib.sv_vat_labels, self.desc,
                                  [None] * 9 + [0, None], "sv_vat_labels")
        if workspace is None:
            workspace = _WS.get(device, nbytes)
        elif workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: need %d bytes" % nbytes)
        self.accept_mask = torch.empty((N, k), dtype=torch.uint8, device=device)
        self.first_reject = torch.empty(N, dtype=torch.int32, device=device)
        self.weights = torch.empty((N, k), dtype=torch.float32, device=device)
        self.probs = torch.empty((N, k, 2), dtype=torch.float32, device=device) if return_probs else None
        rows = N * k * (1 if greedy else 2)
        self.row_stats = torch.empty((rows, 2), dtype=torch.float32, device=device) if return_row_stats else None
        self._keep = (target, draft, draft_tokens, uniforms, workspace)
        self._lib = lib
        self._device = device
        self._head = (ctypes.byref(self.desc), _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                      _ptr(self.accept_mask), _ptr(self.first_reject), _ptr(self.weights), _ptr(self.probs))
        self._ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
        self.set_probe(probe)

    def set_probe(self, probe) -> None:
        self.probe = _probe_ref(probe)

    def __call__(self, stream: Optional[int] = None) -> VatOutput:
        s = _stream_handle(self._device) if stream is None else stream
        if self.row_stats is None and self.probe is None:
            st = self._lib.sv_vat_labels(*self._head, *self._ws, s)
            name = "sv_vat_labels"
        else:
            st = self._lib.sv_vat_labels_ex(*self._head, _ptr(self.row_stats),
                                            None if self.probe is None else ctypes.byref(self.probe), *self._ws, s)
            name = "sv_vat_labels_ex"
        if st:
            raise SVError(st, name, self._lib)
        return VatOutput(self.accept_mask, self.first_reject, self.weights, self.probs, self.row_stats)


def vat_labels(target, draft, draft_tokens, uniforms, temperature: float, decay: float = 0.8, *,
               return_probs: bool = False, return_row_stats: bool = False, workspace=None) -> VatOutput:
    """sv_vat_labels on torch tensors: target/draft [N][k][V], tokens/uniforms [N][k]."""
    return VatLabeler(target, draft, draft_tokens, uniforms, temperature, decay, return_probs=return_probs,
                      return_row_stats=return_row_stats, workspace=workspace)()


class VatLossOutput(NamedTuple):
    accept_mask: "object"
    first_reject: "object"
    weights: "object"
    soft_ce: "object"
    hard_ce: "object"
    block_loss: "object"
    probs: "object"
    row_stats: "object"


class VatLoss:
    """A prepared sv_vat_loss call (see :class:`Verifier`)."""

    def __init__(self, target, draft, draft_tokens, uniforms, hard_tokens, temperature: float, decay: float = 0.8,
                 hard_weight: float = 1.0, *, return_probs: bool = False, return_row_stats: bool = False,
                 workspace=None, probe=None):
        torch = _torch()
        lib = load_library()
        if target.dim() != 3:
            raise ValueError("target must be [N][k][V]")
        N, k, V = (int(s) for s in target.shape)
        device = target.device
        dt = _dtype_code(target)
        _check_dev("target", target, device)
        _check_dev("draft", draft, device, target.dtype, (N, k, V))
        _check_dev("draft_tokens", draft_tokens, device, torch.int32, (N, k))
        _check_dev("uniforms", uniforms, device, torch.float32, (N, k))
        _check_dev("hard_tokens", hard_tokens, device, torch.int32, (N, k))
        self.desc = VatLossDesc(N, k, V, dt, float(temperature), float(decay), float(hard_weight))
        nbytes = _workspace_bytes(lib, lib.sv_vat_loss_workspace_bytes, lib.sv_vat_loss, self.desc,
                                  [None] * 15 + [0, None], "sv_vat_loss")
        if workspace is None:
            workspace = _WS.get(device, nbytes)
        elif workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: need %d bytes" % nbytes)
        self.accept_mask = torch.empty((N, k), dtype=torch.uint8, device=device)
        self.first_reject = torch.empty(N, dtype=torch.int32, device=device)
        self.weights = torch.empty((N, k), dtype=torch.float32, device=device)
        self.soft_ce = torch.empty((N, k), dtype=torch.float32, device=device)
        self.hard_ce = torch.empty((N, k), dtype=torch.float32, device=device)
        self.block_loss = torch.empty(N, dtype=torch.float32, device=device)
        self.probs = torch.empty((N, k, 2), dtype=torch.float32, device=device) if return_probs else None
        self.row_stats = (torch.empty((2 * N * k, 2), dtype=torch.float32, device=device)
                          if return_row_stats else None)
        self._keep = (target, draft, draft_tokens, uniforms, hard_tokens, workspace)
        self._lib = lib
        self._device = device
        self._args = (ctypes.byref(self.desc), _ptr(target), _ptr(draft), _ptr(draft_tokens), _ptr(uniforms),
                      _ptr(hard_tokens), _ptr(self.accept_mask), _ptr(self.first_reject), _ptr(self.weights),
                      _ptr(self.soft_ce), _ptr(self.hard_ce), _ptr(self.block_loss), _ptr(self.probs),
                      _ptr(self.row_stats))
        self._ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
        self.set_probe(probe)

    def set_probe(self, probe) -> None:
        self.probe = _probe_ref(probe)

    def __call__(self, stream: Optional[int] = None) -> VatLossOutput:
        s = _stream_handle(self._device) if stream is None else stream
        st = self._lib.sv_vat_loss(*self._args, None if self.probe is None else ctypes.byref(self.probe),
                                   *self._ws, s)
        if st:
            raise SVError(st, "sv_vat_loss", self._lib)
        return VatLossOutput(self.accept_mask, self.first_reject, self.weights, self.soft_ce, self.hard_ce,
                             self.block_loss, self.probs, self.row_stats)


def vat_loss(target, draft, draft_tokens, uniforms, hard_tokens, temperature: float, decay: float = 0.8,
             hard_weight: float = 1.0, *, return_probs: bool = False, return_row_stats: bool = False,
             workspace=None) -> VatLossOutput:
    """sv_vat_loss on torch tensors: target/draft [N][k][V]; draft tokens, uniforms and hard tokens [N][k].
    Labels, weights, the soft and hard terms per position and the weighted loss per block."""
    return VatLoss(target, draft, draft_tokens, uniforms, hard_tokens, temperature, decay, hard_weight,
                   return_probs=return_probs, return_row_stats=return_row_stats, workspace=workspace)()


class VatLossGrad:
    """A prepared sv_vat_loss_grad call: d(block loss)/d(draft logits), [N][k][V] float32, from the logits and
    what sv_vat_loss wrote for them (weights, row statistics)."""

    def __init__(self, target, draft, hard_tokens, weights, row_stats, temperature: float, hard_weight: float = 1.0,
                 *, out=None, probe=None):
        torch = _torch()
        lib = load_library()
        if target.dim() != 3:
            raise ValueError("target must be [N][k][V]")
        N, k, V = (int(s) for s in target.shape)
        device = target.device
        dt = _dtype_code(target)
        _check_dev("target", target, device)
        _check_dev("draft", draft, device, target.dtype, (N, k, V))
        _check_dev("hard_tokens", hard_tokens, device, torch.int32, (N, k))
        _check_dev("weights", weights, device, torch.float32, (N, k))
        _check_dev("row_stats", row_stats, device, torch.float32, (2 * N * k, 2))
        self.grad = out if out is not None else torch.empty((N, k, V), dtype=torch.float32, device=device)
        _check_dev("out", self.grad, device, torch.float32, (N, k, V))
        self.desc = VatLossDesc(N, k, V, dt, float(temperature), 0.0, float(hard_weight))
        self._keep = (target, draft, hard_tokens, weights, row_stats)
        self._lib = lib
        self._device = device
        self._args = (ctypes.byref(self.desc), _ptr(target), _ptr(draft), _ptr(hard_tokens), _ptr(weights),
                      _ptr(row_stats), _ptr(self.grad))
        self.set_probe(probe)

    def set_probe(self, probe) -> None:
        self.probe = _probe_ref(probe)

    def __call__(self, stream: Optional[int] = None):
        s = _stream_handle(self._device) if stream is None else stream
        st = self._lib.sv_vat_loss_grad(*self._args, None if self.probe is None else ctypes.byref(self.probe), s)
        if st:
            raise SVError(st, "sv_vat_loss_grad", self._lib)
        return self.grad


def vat_loss_grad(target, draft, hard_tokens, weights, row_stats, temperature: float, hard_weight: float = 1.0,
                  *, out=None):
    """sv_vat_loss_grad on torch tensors: the gradient of vat_loss's block losses with respect to the draft
    logits, given the weights and row statistics vat_loss returned (return_row_stats=True)."""
    return VatLossGrad(target, draft, hard_tokens, weights, row_stats, temperature, hard_weight, out=out)()


class LmHeadOutput(NamedTuple):
    accepted_len: "object"
    out_tokens: "object"
    argmax: "object"


class LmHeadVerifier:
    """A prepared sv_verify_lm_head_greedy call (greedy verification with the
    target's logits formed from its hidden states inside the call)."""

    def __init__(self, hidden_states, weight, draft_tokens, *, return_argmax: bool = False, workspace=None,
                 probe=None):
        torch = _torch()
        lib = load_library()
        if hidden_states.dim() != 3 or weight.dim() != 2:
            raise ValueError("hidden_states must be [B][k+1][D] and weight [V][D]")
        B, kp1, D = (int(s) for s in hidden_states.shape)
        k = kp1 - 1
        V = int(weight.shape[0])
        device = hidden_states.device
        _check_dev("hidden_states", hidden_states, device, torch.bfloat16)
        _check_dev("weight", weight, device, torch.bfloat16, (V, D))
        _check_dev("draft_tokens", draft_tokens, device, torch.int32, (B, k))
        self.desc = LmHeadDesc(B, k, V, D)
        nbytes = _workspace_bytes(lib, lib.sv_lm_head_workspace_bytes, lib.sv_verify_lm_head_greedy, self.desc,
                                  [None] * 8 + [0, None], "sv_verify_lm_head_greedy")
        if workspace is None:
            workspace = _WS_LM.get(device, nbytes)
        elif workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: need %d bytes" % nbytes)
        self.accepted_len = torch.empty(B, dtype=torch.int32, device=device)
        self.out_tokens = torch.empty((B, k + 1), dtype=torch.int32, device=device)
        self.argmax = torch.empty((B, k + 1), dtype=torch.int32, device=device) if return_argmax else None
        self._keep = (hidden_states, weight, draft_tokens, workspace)
        self._lib = lib
        self._device = device
        self._args = (ctypes.byref(self.desc), _ptr(hidden_states), _ptr(weight), _ptr(draft_tokens),
                      _ptr(self.accepted_len), _ptr(self.out_tokens), _ptr(self.argmax))
        self._ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
        self.set_probe(probe)

    def set_probe(self, probe) -> None:
        self.probe = _probe_ref(probe)

    def __call__(self, stream: Optional[int] = None) -> LmHeadOutput:
        s = _stream_handle(self._device) if stream is None else stream
        st = self._lib.sv_verify_lm_head_greedy(*self._args, None if self.probe is None else ctypes.byref(self.probe),
                                                *self._ws, s)
        if st:
            raise SVError(st, "sv_verify_lm_head_greedy", self._lib)
        return LmHeadOutput(self.accepted_len, self.out_tokens, self.argmax)


def verify_lm_head_greedy(hidden_states, weight, draft_tokens, *, return_argmax: bool = False,
                          workspace=None) -> LmHeadOutput:
    """sv_verify_lm_head_greedy on torch tensors: hidden_states [B][k+1][D]
    bf16, weight [V][D] bf16, draft_tokens [B][k] int32.  Returns
    (accepted_len [B], out_tokens [B][k+1], argmax [B][k+1] or None)."""
    return LmHeadVerifier(hidden_states, weight, draft_tokens, return_argmax=return_argmax,
                          workspace=workspace)()


class LmHeadSampleOutput(NamedTuple):
    accepted_len: "object"
    out_tokens: "object"
    probs: "object"


class LmHeadSampler:
    """A prepared sv_verify_lm_head call (T > 0: both distributions formed
    from hidden states inside the call)."""

    def __init__(self, target_hidden, target_weight, draft_hidden, draft_weight, draft_tokens, uniforms,
                 temperature: float, *, return_probs: bool = False, workspace=None, probe=None):
        torch = _torch()
        lib = load_library()
        if target_hidden.dim() != 3 or target_weight.dim() != 2:
            raise ValueError("target_hidden must be [B][k+1][D] and target_weight [V][D]")
        B, kp1, D = (int(s) for s in target_hidden.shape)
        k = kp1 - 1
        V = int(target_weight.shape[0])
        device = target_hidden.device
        _check_dev("target_hidden", target_hidden, device, torch.bfloat16)
        _check_dev("target_weight", target_weight, device, torch.bfloat16, (V, D))
        _check_dev("draft_hidden", draft_hidden, device, torch.bfloat16, (B, k, D))
        _check_dev("draft_weight", draft_weight, device, torch.bfloat16, (V, D))
        _check_dev("draft_tokens", draft_tokens, device, torch.int32, (B, k))
        _check_dev("uniforms", uniforms, device, torch.float32, (B, k + 1))
        self.desc = LmHeadSampleDesc(B, k, V, D, float(temperature))
        nbytes = _workspace_bytes(lib, lib.sv_lm_head_sample_workspace_bytes, lib.sv_verify_lm_head, self.desc,
                                  [None] * 11 + [0, None], "sv_verify_lm_head")
        if workspace is None:
            workspace = _WS_LM.get(device, nbytes)
        elif workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small: need %d bytes" % nbytes)
        self.accepted_len = torch.empty(B, dtype=torch.int32, device=device)
        self.out_tokens = torch.empty((B, k + 1), dtype=torch.int32, device=device)
        self.probs = torch.empty((B, k, 2), dtype=torch.float32, device=device) if return_probs else None
        self._keep = (target_hidden, target_weight, draft_hidden, draft_weight, draft_tokens, uniforms, workspace)
        self._lib = lib
        self._device = device
        self._args = (ctypes.byref(self.desc), _ptr(target_hidden), _ptr(target_weight), _ptr(draft_hidden),
                      _ptr(draft_weight), _ptr(draft_tokens), _ptr(uniforms), _ptr(self.accepted_len),
                      _ptr(self.out_tokens), _ptr(self.probs))
        self._ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
        self.set_probe(probe)

    def set_probe(self, probe) -> None:
        self.probe = _probe_ref(probe)

    def __call__(self, stream: Optional[int] = None) -> LmHeadSampleOutput:
        s = _stream_handle(self._device) if stream is None else stream
        st = self._lib.sv_verify_lm_head(*self._args, None if self.probe is None else ctypes.byref(self.probe),
                                         *self._ws, s)
        if st:
            raise SVError(st, "sv_verify_lm_head", self._lib)
        return LmHeadSampleOutput(self.accepted_len, self.out_tokens, self.probs)


def verify_lm_head(target_hidden, target_weight, draft_hidden, draft_weight, draft_tokens, uniforms,
                   temperature: float, *, return_probs: bool = False, workspace=None) -> LmHeadSampleOutput:
    """sv_verify_lm_head on torch tensors (bf16 hidden states and weights,
    int32 tokens, float32 uniforms [B][k+1]).  Returns (accepted_len [B],
    out_tokens [B][k+1], probs [B][k][2] or None)."""
    return LmHeadSampler(target_hidden, target_weight, draft_hidden, draft_weight, draft_tokens, uniforms,
                         temperature, return_probs=return_probs, workspace=workspace)()


def accept_histogram(accepted_len, k: int, out=None, stream: Optional[int] = None):
    """sv_accept_histogram: counts of accepted lengths 0..k, then -1, -2 and
    other values, as an int32 tensor of k+4 on the same device."""
    torch = _torch()
    lib = load_library()
    device = accepted_len.device
    _check_dev("accepted_len", accepted_len, device, torch.int32)
    if out is None:
        out = torch.empty(k + 4, dtype=torch.int32, device=device)
    _check_dev("out", out, device, torch.int32, (k + 4,))
    s = _stream_handle(device) if stream is None else stream
    st = lib.sv_accept_histogram(_ptr(accepted_len), int(accepted_len.numel()), int(k), _ptr(out), s)
    if st:
        raise SVError(st, "sv_accept_histogram", lib)
    return out


def sol_read(data, sink, stream: Optional[int] = None) -> None:
    """sv_sol_read over the bytes of a contiguous device tensor (a multiple
    of 16 bytes, 16-byte aligned); sink: a device int32/uint32 tensor of at
    least one element."""
    lib = load_library()
    if not data.is_contiguous() or sink.device != data.device:
        raise ValueError("sol_read: contiguous data and a sink on the same device")
    s = _stream_handle(data.device) if stream is None else stream
    st = lib.sv_sol_read(_ptr(data), data.numel() * data.element_size(), _ptr(sink), s)
    if st:
        raise SVError(st, "sv_sol_read", lib)


def sol_read_write(a, b, out, stream: Optional[int] = None) -> None:
    """sv_sol_read_write: out = a - b in fp32 (a, b float32 or bfloat16 of the
    same length as the float32 `out`, all contiguous on one device)."""
    torch = _torch()
    lib = load_library()
    device = a.device
    _check_dev("b", b, device, a.dtype, tuple(a.shape))
    _check_dev("out", out, device, torch.float32)
    if not a.is_contiguous() or out.numel() != a.numel():
        raise ValueError("sol_read_write: contiguous operands of one length")
    s = _stream_handle(device) if stream is None else stream
    st = lib.sv_sol_read_write(_ptr(a), _ptr(b), _ptr(out), a.numel(), _dtype_code(a), s)
    if st:
        raise SVError(st, "sv_sol_read_write", lib)


class DraftLengthController:
    """The host-side draft-length rule (sv_draft_len_init / sv_draft_len_update):
    choices ascending (default 5, 7, 9, 11), start at the shortest, move one
    step up or down after `patience` consecutive steps whose block efficiency
    is at least up_frac*(k+1) or at most down_frac*(k+1).  `lib`: a ctypes
    library exporting the two controller symbols (default: libspecverify)."""

    def __init__(self, choices=(5, 7, 9, 11), up_frac: float = 0.9, down_frac: float = 0.5, patience: int = 2,
                 lib=None):
        if lib is None:
            lib = load_library()
        else:
            _bind_control(lib)
        self._lib = lib
        self.ctl = DraftLenCtl()
        arr = (ctypes.c_int32 * len(choices))(*choices)
        st = lib.sv_draft_len_init(ctypes.byref(self.ctl), arr, len(choices), float(up_frac), float(down_frac),
                                   int(patience))
        if st:
            raise SVError(st, "sv_draft_len_init", lib)

    @property
    def k(self) -> int:
        return int(self.ctl.choices[self.ctl.index])

    @property
    def efficiency(self) -> float:
        return float(self.ctl.last_efficiency)

    def update(self, hist) -> int:
        """hist: host sequence (or tensor) of the k+4 counts for a step run at
        the current k.  Returns the draft length for the next step."""
        vals = [int(v) for v in (hist.tolist() if hasattr(hist, "tolist") else hist)]
        if len(vals) < self.k + 1:
            raise ValueError("hist needs at least k+1 = %d counts" % (self.k + 1))
        arr = (ctypes.c_int32 * len(vals))(*vals)
        nxt = ctypes.c_int32()
        st = self._lib.sv_draft_len_update(ctypes.byref(self.ctl), arr, self.k, ctypes.byref(nxt))
        if st:
            raise SVError(st, "sv_draft_len_update", self._lib)
        return int(nxt.value)
