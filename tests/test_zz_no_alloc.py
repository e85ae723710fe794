"""sv_verify_noalloc (the entry point that allocates nothing: its workspace is
an array built into the library) against sv_verify on the same inputs,
through the C ABI: two calls in a row on one device, the second smaller, each
compared element by element with sv_verify's outputs (bit for bit: the same
kernels run on the same inputs).  Also the host-side rejection of a call that
needs more than the built-in workspace."""
import ctypes

import numpy as np
import pytest

import speculative_decoding_verification_amd as sv
import workloads

pytestmark = pytest.mark.gpu


def _noalloc(lib, t, d, x, u, T, onehot, stream):
    import torch

    B, kp1, V = (int(s) for s in t.shape)
    k = kp1 - 1
    desc = sv.VerifyDesc(B, k, V, sv.SV_BF16 if t.dtype == torch.bfloat16 else sv.SV_F32,
                         sv.SV_DRAFT_ONEHOT if onehot else sv.SV_DRAFT_LOGITS, float(T))
    acc = torch.full((B,), 12345, dtype=torch.int32, device=t.device)
    out = torch.full((B, k + 1), 12345, dtype=torch.int32, device=t.device)
    probs = torch.full((B, k, 2), float("nan"), dtype=torch.float32, device=t.device)
    uses_draft = not onehot and T != 0.0
    st = lib.sv_verify_noalloc(ctypes.byref(desc), t.data_ptr(), d.data_ptr() if uses_draft else None,
                               x.data_ptr(), u.data_ptr() if T != 0.0 else None, acc.data_ptr(), out.data_ptr(),
                               probs.data_ptr(), stream)
    assert st == 0, lib.sv_status_str(st).decode()
    return acc, out, probs


@pytest.mark.parametrize("first,second", [
    (("selfdraft", dict(B=24)), ("selfdraft", dict(B=5))),
    (("ngram_tail", dict(B=8)), ("tiny", dict())),
    (("grpo_greedy", dict(B=40)), ("grpo_greedy", dict(B=3))),
])
def test_noalloc_matches_verify_on_two_calls(first, second):
    import torch

    lib = sv.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    for name, scale in (first, second):
        cfg = workloads.get_config(name).scaled(**scale) if scale else workloads.get_config(name)
        print("noalloc case:", name, scale, flush=True)
        wl = workloads.generate(cfg)
        t, d, x, u = workloads.to_device(wl, dev)
        ref = sv.verify(t, d, x, u, cfg.T, onehot=cfg.onehot, return_probs=True)
        acc, out, probs = _noalloc(lib, t, d, x, u, cfg.T, cfg.onehot, stream)
        torch.cuda.synchronize()
        assert torch.equal(acc, ref.accepted_len)
        assert torch.equal(out, ref.out_tokens)
        assert torch.equal(probs.view(torch.int32), ref.probs.view(torch.int32))
        assert int((acc < 0).sum()) == 0


def test_noalloc_binding_and_scratch_limit():
    import torch

    lib = sv.load_library()
    dev = torch.device("cuda:0")
    cfg = workloads.get_config("selfdraft").scaled(B=3)
    wl = workloads.generate(cfg)
    t, d, x, u = workloads.to_device(wl, dev)
    a = sv.verify_noalloc(t, d, x, u, cfg.T)
    b = sv.verify(t, d, x, u, cfg.T)
    torch.cuda.synchronize()
    assert torch.equal(a.accepted_len, b.accepted_len) and torch.equal(a.out_tokens, b.out_tokens)
    # a call whose hand-off words exceed the built-in workspace is refused on
    # the host before anything is launched (no device pointer is touched)
    big = sv.VerifyDesc(4096, 16, 151936, sv.SV_BF16, sv.SV_DRAFT_LOGITS, 1.0)
    assert lib.sv_verify_workspace_bytes(ctypes.byref(big)) > 8 << 20
    st = lib.sv_verify_noalloc(ctypes.byref(big), 16, 16, 16, 16, 16, 16, None, None)
    assert st == 13
