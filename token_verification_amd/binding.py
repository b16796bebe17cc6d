"""ctypes binding of libspecverify.so (argument marshalling only).

Every step of the verify computation runs in the HIP library; this module
checks the dtypes, shapes, devices and layout of every input and of any
caller-supplied output or workspace tensor (ValueError on a mismatch),
allocates outputs, keeps one workspace per (device, stream), and passes raw
device pointers plus the current stream to the C ABI declared in
``include/spec_verify.h``.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import NamedTuple, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SAMPLE = 0
GREEDY = 1
MARGIN = 0          # spec_gate: fire iff gap > tau
CERTIFIED = 1       # spec_gate: fire iff gap > 0 and 2 * tau <= gap
F32 = 0
BF16 = 1

_ERRORS = {
    -1: "SPEC_ERR_NULL", -2: "SPEC_ERR_SHAPE", -3: "SPEC_ERR_DTYPE", -4: "SPEC_ERR_MODE",
    -5: "SPEC_ERR_TEMP", -6: "SPEC_ERR_WORKSPACE", -7: "SPEC_ERR_ALIGN", -8: "SPEC_ERR_HIP",
    -9: "SPEC_ERR_VALUE",
}


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERRORS.get(code, code)}: {msg}")
        self.code = code


_lib = None
_lock = threading.Lock()


def lib():
    """The loaded HIP library. Raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise SpecVerifyError(
                        -8, f"{LIB_PATH} is missing: build it with `python -m token_verification_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                P, I, F, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
                L.spec_verify.argtypes = [P, P, P, P, F, ctypes.c_int, I, I, I, ctypes.c_int,
                                          P, P, P, P, P, P, S, P]
                L.spec_verify.restype = ctypes.c_int
                L.spec_verify_ragged.argtypes = [P, P, P, P, P, F, ctypes.c_int, I, I, I, ctypes.c_int,
                                                 P, P, P, P, P, P, S, P]
                L.spec_verify_ragged.restype = ctypes.c_int
                L.spec_verify_timed.argtypes = [P, P, P, P, P, F, ctypes.c_int, I, I, I, ctypes.c_int,
                                                P, P, P, P, P, P, S, P, P]
                L.spec_verify_timed.restype = ctypes.c_int
                L.spec_verify_noalloc.argtypes = [P, P, P, P, F, ctypes.c_int, I, I, I, ctypes.c_int,
                                                  P, P, P, P, P, P]
                L.spec_verify_noalloc.restype = ctypes.c_int
                L.spec_verify_workspace_size.argtypes = [I, I, I, ctypes.c_int, ctypes.c_int]
                L.spec_verify_workspace_size.restype = S
                L.spec_verify_check_args.argtypes = [P, P, P, P, F, ctypes.c_int, I, I, I, ctypes.c_int,
                                                     P, P, P, P, S]
                L.spec_verify_check_args.restype = ctypes.c_int
                L.spec_gate.argtypes = [P, I, I, ctypes.c_int, ctypes.c_int, F, P, P, P, P, P, S, P]
                L.spec_gate.restype = ctypes.c_int
                L.spec_gate_workspace_size.argtypes = [I, I, ctypes.c_int]
                L.spec_gate_workspace_size.restype = S
                L.spec_commit.argtypes = [P, I, I, P, P, P, S, P]
                L.spec_commit.restype = ctypes.c_int
                L.spec_verify_lmhead.argtypes = [P, P, P, P, P, I, I, I, I, P, P, P, P, S, P]
                L.spec_verify_lmhead.restype = ctypes.c_int
                L.spec_verify_lmhead_timed.argtypes = [P, P, P, P, P, I, I, I, I, P, P, P, P, S, P, P]
                L.spec_verify_lmhead_timed.restype = ctypes.c_int
                L.spec_lmhead_workspace_size.argtypes = [I, I, I, I]
                L.spec_lmhead_workspace_size.restype = S
                L.spec_verify_lmhead_sample.argtypes = [P, P, P, P, P, P, P, P, P, P, F, I, I, I, I,
                                                        P, P, P, P, P, P, S, P]
                L.spec_verify_lmhead_sample.restype = ctypes.c_int
                L.spec_verify_lmhead_sample_timed.argtypes = [P, P, P, P, P, P, P, P, P, P, F, I, I, I, I,
                                                              P, P, P, P, P, P, S, P, P]
                L.spec_verify_lmhead_sample_timed.restype = ctypes.c_int
                L.spec_lmhead_sample_workspace_size.argtypes = [I, I, I, I]
                L.spec_lmhead_sample_workspace_size.restype = S
                L.spec_lmhead_packed_size.argtypes = [I, I]
                L.spec_lmhead_packed_size.restype = S
                L.spec_lmhead_pack.argtypes = [P, I, I, P, S, P]
                L.spec_lmhead_pack.restype = ctypes.c_int
                L.spec_verify_lmhead_packed.argtypes = [P, P, P, P, P, I, I, I, I, P, P, P, P, S, P, P]
                L.spec_verify_lmhead_packed.restype = ctypes.c_int
                L.spec_verify_lmhead_sample_packed.argtypes = list(L.spec_verify_lmhead_sample_timed.argtypes)
                L.spec_verify_lmhead_sample_packed.restype = ctypes.c_int
                L.spec_verify_last_error.restype = ctypes.c_char_p
                L.spec_verify_version.restype = ctypes.c_char_p
                _lib = L
    return _lib


def last_error() -> str:
    return lib().spec_verify_last_error().decode()


def workspace_size(B: int, k: int, V: int, dtype: int, mode: int) -> int:
    return int(lib().spec_verify_workspace_size(B, k, V, dtype, mode))


def check_args(target_ptr, draft_ptr, tokens_ptr, uniforms_ptr, temperature, mode, B, k, V, dtype,
               acc_ptr, out_ptr, gap_ptr, ws_ptr, ws_bytes) -> int:
    """Host-only argument check on raw pointer values (no HIP call)."""
    return int(lib().spec_verify_check_args(target_ptr, draft_ptr, tokens_ptr, uniforms_ptr,
                                            ctypes.c_float(temperature), mode, B, k, V, dtype,
                                            acc_ptr, out_ptr, gap_ptr, ws_ptr, ws_bytes))


class VerifyResult(NamedTuple):
    accepted_len: torch.Tensor   # [B] int32
    out_tokens: torch.Tensor     # [B, k+1] int32
    gap: torch.Tensor            # [B, k+1] float32
    target_prob: Optional[torch.Tensor]   # [B, k] float32 or None
    draft_prob: Optional[torch.Tensor]


_ws_cache: dict = {}
_need_cache: dict = {}


def _workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    """One workspace per (device, stream); every record in it is written before
    it is read, so it needs no initialisation."""
    key = (device.index, stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _user_workspace(ws: torch.Tensor, device: torch.device, nbytes: int) -> torch.Tensor:
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {nbytes}")
    return ws


def _check_out_tensor(t, name: str, shape, dtype, device: torch.device) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"out.{name} must be a tensor")
    if tuple(t.shape) != shape or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"out.{name} must be a contiguous {dtype} tensor of shape {list(shape)} on {device} "
                         f"(got {t.dtype} {list(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ', not contiguous'})")


def _check_out(out, B: int, k: int, device: torch.device, probs: bool) -> None:
    """Every output tensor the library will write: shape, dtype, device, layout."""
    if not isinstance(out, VerifyResult):
        raise ValueError("out must be a VerifyResult")
    _check_out_tensor(out.accepted_len, "accepted_len", (B,), torch.int32, device)
    _check_out_tensor(out.out_tokens, "out_tokens", (B, k + 1), torch.int32, device)
    _check_out_tensor(out.gap, "gap", (B, k + 1), torch.float32, device)
    if probs and (out.target_prob is None or out.draft_prob is None):
        raise ValueError("return_probs=True needs out.target_prob and out.draft_prob")
    for name in ("target_prob", "draft_prob"):
        t = getattr(out, name)
        if t is not None:
            _check_out_tensor(t, name, (B, k), torch.float32, device)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def spec_verify(target: torch.Tensor, draft: Optional[torch.Tensor], tokens: torch.Tensor,
                uniforms: Optional[torch.Tensor], temperature: float = 1.0, mode: int = SAMPLE, *,
                workspace: Optional[torch.Tensor] = None, return_probs: bool = False,
                out: Optional[VerifyResult] = None,
                draft_len: Optional[torch.Tensor] = None,
                phase_events=None) -> VerifyResult:
    """Batched verify step on device tensors (see include/spec_verify.h).

    target [B,k+1,V] and draft [B,k,V] are float32 or bfloat16 (draft may be
    None in greedy mode), tokens [B,k] int32, uniforms [B,k+1,2] float32 (None
    allowed in greedy mode). With draft_len (int32 [B] on the same device)
    every batch row b verifies only its first draft_len[b] positions
    (spec_verify_ragged). With phase_events (four torch.cuda.Event created
    with enable_timing=True) the call goes through spec_verify_timed, which
    records them before pass 1, after pass 1, after pass 2 and after the draw.
    Work is enqueued on the current stream of the target's device; the
    returned tensors are ready once that stream is.
    """
    if not isinstance(target, torch.Tensor) or target.dim() != 3:
        raise ValueError("target must be a [B, k+1, V] tensor")
    if not target.is_cuda:
        raise ValueError("target must be a device tensor")
    if target.dtype == torch.float32:
        dtype = F32
    elif target.dtype == torch.bfloat16:
        dtype = BF16
    else:
        raise ValueError(f"unsupported logit dtype {target.dtype}")
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    if draft is not None:
        if draft.shape != (B, k, V) or draft.dtype != target.dtype or draft.device != dev:
            raise ValueError("draft must match target's dtype/device with shape [B, k, V]")
    if tokens.shape != (B, k) or tokens.dtype != torch.int32 or tokens.device != dev:
        raise ValueError("tokens must be int32 [B, k] on the target's device")
    if uniforms is not None:
        if uniforms.shape != (B, k + 1, 2) or uniforms.dtype != torch.float32 or uniforms.device != dev:
            raise ValueError("uniforms must be float32 [B, k+1, 2] on the target's device")
    if draft_len is not None:
        if draft_len.shape != (B,) or draft_len.dtype != torch.int32 or draft_len.device != dev:
            raise ValueError("draft_len must be int32 [B] on the target's device")
    for t in (target, draft, tokens, uniforms, draft_len):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")

    if out is None:
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        otok = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
        gap = torch.empty((B, k + 1), dtype=torch.float32, device=dev)
        tp = torch.empty((B, k), dtype=torch.float32, device=dev) if return_probs else None
        dp = torch.empty((B, k), dtype=torch.float32, device=dev) if return_probs else None
        out = VerifyResult(acc, otok, gap, tp, dp)
    else:
        _check_out(out, B, k, dev, return_probs)

    stream = torch.cuda.current_stream(dev).cuda_stream
    nkey = (B, k, V, dtype, int(mode))
    need = _need_cache.get(nkey)
    if need is None:
        need = workspace_size(B, k, V, dtype, mode)
        if need == 0:
            raise SpecVerifyError(-2, f"unsupported sizes B={B} k={k} V={V}")
        _need_cache[nkey] = need
    ws = _workspace(dev, stream, need) if workspace is None else _user_workspace(workspace, dev, need)
    tail = (ctypes.c_float(temperature), int(mode), B, k, V, dtype,
            _ptr(out.accepted_len), _ptr(out.out_tokens), _ptr(out.gap),
            _ptr(out.target_prob), _ptr(out.draft_prob),
            ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), ctypes.c_void_p(stream))
    if phase_events is not None:
        if len(phase_events) != 4:
            raise ValueError("phase_events must hold four events")
        handles = []
        for ev in phase_events:
            if not ev.cuda_event:                         # torch creates events lazily
                ev.record(torch.cuda.current_stream(dev))
            handles.append(ev.cuda_event)
        arr = (ctypes.c_void_p * 4)(*handles)
        rc = lib().spec_verify_timed(_ptr(target), _ptr(draft), _ptr(tokens), _ptr(draft_len), _ptr(uniforms),
                                     *tail, ctypes.cast(arr, ctypes.c_void_p))
    elif draft_len is None:
        rc = lib().spec_verify(_ptr(target), _ptr(draft), _ptr(tokens), _ptr(uniforms), *tail)
    else:
        rc = lib().spec_verify_ragged(_ptr(target), _ptr(draft), _ptr(tokens), _ptr(draft_len),
                                      _ptr(uniforms), *tail)
    if rc != 0:
        raise SpecVerifyError(rc, last_error())
    return out


def spec_verify_noalloc(target: torch.Tensor, draft: Optional[torch.Tensor], tokens: torch.Tensor,
                        uniforms: Optional[torch.Tensor], temperature: float = 1.0, mode: int = SAMPLE, *,
                        return_probs: bool = False, out: Optional[VerifyResult] = None) -> VerifyResult:
    """spec_verify through spec_verify_noalloc: the library's own device scratch
    serves as the workspace, so the call allocates nothing when ``out`` is
    given (see include/spec_verify.h; calls that overlap on one GPU race)."""
    if not isinstance(target, torch.Tensor) or target.dim() != 3 or not target.is_cuda:
        raise ValueError("target must be a [B, k+1, V] device tensor")
    if target.dtype == torch.float32:
        dtype = F32
    elif target.dtype == torch.bfloat16:
        dtype = BF16
    else:
        raise ValueError(f"unsupported logit dtype {target.dtype}")
    B, k1, V = target.shape
    k = k1 - 1
    dev = target.device
    if draft is not None and (draft.shape != (B, k, V) or draft.dtype != target.dtype or draft.device != dev):
        raise ValueError("draft must match target's dtype/device with shape [B, k, V]")
    if tokens.shape != (B, k) or tokens.dtype != torch.int32 or tokens.device != dev:
        raise ValueError("tokens must be int32 [B, k] on the target's device")
    if uniforms is not None and (uniforms.shape != (B, k + 1, 2) or uniforms.dtype != torch.float32
                                 or uniforms.device != dev):
        raise ValueError("uniforms must be float32 [B, k+1, 2] on the target's device")
    for t in (target, draft, tokens, uniforms):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                           torch.empty((B, k + 1), dtype=torch.float32, device=dev),
                           torch.empty((B, k), dtype=torch.float32, device=dev) if return_probs else None,
                           torch.empty((B, k), dtype=torch.float32, device=dev) if return_probs else None)
    else:
        _check_out(out, B, k, dev, return_probs)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().spec_verify_noalloc(_ptr(target), _ptr(draft), _ptr(tokens), _ptr(uniforms),
                                   ctypes.c_float(temperature), int(mode), B, k, V, dtype,
                                   _ptr(out.accepted_len), _ptr(out.out_tokens), _ptr(out.gap),
                                   _ptr(out.target_prob), _ptr(out.draft_prob), ctypes.c_void_p(stream))
    if rc != 0:
        raise SpecVerifyError(rc, last_error())
    return out


class GateResult(NamedTuple):
    argmax: torch.Tensor   # [n] int32, -1 for an invalid row
    gap: torch.Tensor      # [n] float32
    fire: torch.Tensor     # [n] int32 (0/1)


def spec_gate(logits: torch.Tensor, tau: float = 2.0, admit: Optional[torch.Tensor] = None,
              rule: int = MARGIN, *, workspace: Optional[torch.Tensor] = None,
              out: Optional[GateResult] = None) -> GateResult:
    """Confidence gate over the rows of logits [n, V] (see include/spec_verify.h).

    admit: optional int32/uint32-sized bit mask [(V + 31) // 32] of admissible
    tokens on the same device (int32 tensors carry the bits unchanged).
    """
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2 or not logits.is_cuda:
        raise ValueError("logits must be a [n, V] device tensor")
    if logits.dtype == torch.float32:
        dtype = F32
    elif logits.dtype == torch.bfloat16:
        dtype = BF16
    else:
        raise ValueError(f"unsupported logit dtype {logits.dtype}")
    n, V = logits.shape
    dev = logits.device
    if admit is not None:
        if admit.shape != ((V + 31) // 32,) or admit.element_size() != 4 or admit.device != dev:
            raise ValueError("admit must be a 32-bit [(V+31)//32] mask on the logits' device")
    for t in (logits, admit):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = GateResult(torch.empty(n, dtype=torch.int32, device=dev),
                         torch.empty(n, dtype=torch.float32, device=dev),
                         torch.empty(n, dtype=torch.int32, device=dev))
    else:
        if not isinstance(out, GateResult):
            raise ValueError("out must be a GateResult")
        _check_out_tensor(out.argmax, "argmax", (n,), torch.int32, dev)
        _check_out_tensor(out.gap, "gap", (n,), torch.float32, dev)
        _check_out_tensor(out.fire, "fire", (n,), torch.int32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = int(lib().spec_gate_workspace_size(n, V, dtype))
    if need == 0:
        raise SpecVerifyError(-2, f"unsupported sizes n={n} V={V}")
    ws = _workspace(dev, stream, need) if workspace is None else _user_workspace(workspace, dev, need)
    rc = lib().spec_gate(_ptr(logits), n, V, dtype, int(rule), ctypes.c_float(tau), _ptr(admit),
                         _ptr(out.argmax), _ptr(out.gap), _ptr(out.fire),
                         ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), ctypes.c_void_p(stream))
    if rc != 0:
        raise SpecVerifyError(rc, last_error())
    return out


def spec_commit(accepted_len: torch.Tensor, k: int, kv_len: Optional[torch.Tensor] = None,
                slots: Optional[torch.Tensor] = None, state: Optional[torch.Tensor] = None) -> None:
    """Commit a verify step in place (see include/spec_verify.h): kv_len[b] += 1 + a
    and state[b] = slots[b, a] for every row with a = accepted_len[b] in [0, k].

    accepted_len int32 [B]; kv_len int32 [B] or None; slots [B, k+1, ...] and
    state [B, ...] of one dtype (any), or both None.
    """
    if accepted_len.dim() != 1 or accepted_len.dtype != torch.int32 or not accepted_len.is_cuda:
        raise ValueError("accepted_len must be an int32 [B] device tensor")
    B = accepted_len.shape[0]
    dev = accepted_len.device
    if kv_len is not None:
        if kv_len.shape != (B,) or kv_len.dtype != torch.int32 or kv_len.device != dev:
            raise ValueError("kv_len must be int32 [B] on accepted_len's device")
    if (slots is None) != (state is None):
        raise ValueError("slots and state go together")
    row = 0
    if state is not None:
        if state.shape[0] != B or slots.shape[:2] != (B, k + 1) or slots.shape[2:] != state.shape[1:]:
            raise ValueError("slots must be [B, k+1, *S] and state [B, *S]")
        if slots.dtype != state.dtype or slots.device != dev or state.device != dev:
            raise ValueError("slots and state must share a dtype and accepted_len's device")
        row = state[0].numel() * state.element_size() if B else 0
    for t in (accepted_len, kv_len, slots, state):
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib().spec_commit(_ptr(accepted_len), B, int(k), _ptr(kv_len), _ptr(slots), _ptr(state), row,
                           ctypes.c_void_p(stream))
    if rc != 0:
        raise SpecVerifyError(rc, last_error())


class PackedHead(NamedTuple):
    """An int8 LM head [V, d] in the tile-major layout (spec_lmhead_pack)."""
    data: torch.Tensor                                    # int8, spec_lmhead_packed_size(V, d) bytes
    V: int
    d: int


def pack_lmhead(weight: torch.Tensor) -> PackedHead:
    """The tile-major copy of an int8 head weight [V, d] (see include/spec_verify.h),
    written on the current stream; pass it as `weight` / `draft_weight` to
    spec_verify_lmhead and spec_verify_lmhead_sample."""
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2 or weight.dtype != torch.int8 \
            or not weight.is_cuda or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous int8 2-D device tensor")
    V, d = weight.shape
    need = int(lib().spec_lmhead_packed_size(V, d))
    if need == 0:
        raise SpecVerifyError(-2, f"unsupported sizes V={V} d={d}")
    data = torch.empty(need, dtype=torch.int8, device=weight.device)
    stream = torch.cuda.current_stream(weight.device).cuda_stream
    rc = lib().spec_lmhead_pack(_ptr(weight), V, d, _ptr(data), need, ctypes.c_void_p(stream))
    if rc != 0:
        raise SpecVerifyError(rc, last_error())
    return PackedHead(data, int(V), int(d))


def _head_arg(w, d: int, name: str):
    """(tensor to pass, V, packed) for a head given row-major or packed."""
    if isinstance(w, PackedHead):
        t = w.data
        if not isinstance(t, torch.Tensor) or t.dtype != torch.int8 or not t.is_cuda or t.dim() != 1:
            raise ValueError(f"{name}.data must be an int8 1-D device tensor")
        if w.d != d:
            raise ValueError(f"hidden and {name} must share d")
        if t.numel() < int(lib().spec_lmhead_packed_size(w.V, w.d)):
            raise ValueError(f"{name}.data is smaller than the packed head")
        return t, int(w.V), True
    if not isinstance(w, torch.Tensor) or w.dim() != 2 or w.dtype != torch.int8 or not w.is_cuda:
        raise ValueError(f"{name} must be an int8 2-D device tensor or a PackedHead")
    if w.shape[1] != d:
        raise ValueError(f"hidden and {name} must share d")
    return w, int(w.shape[0]), False


def spec_verify_lmhead(hidden: torch.Tensor, hidden_scale: torch.Tensor, weight: torch.Tensor,
                       weight_scale: torch.Tensor, tokens: torch.Tensor, *,
                       workspace: Optional[torch.Tensor] = None, out: Optional[VerifyResult] = None,
                       phase_events=None) -> VerifyResult:
    """Greedy verification fused with an int8 LM head (see include/spec_verify.h).

    hidden int8 [B*(k+1), d] (row b*(k+1)+i: position i of batch row b),
    hidden_scale float32 [B*(k+1)], weight int8 [V, d], weight_scale float32
    [V], tokens int32 [B, k], all on one device; weight may instead be a
    PackedHead (pack_lmhead). With phase_events (three torch.cuda.Event
    created with enable_timing=True) the call records them before the LM-head
    kernel, after it and after the decisions.
    """
    if not isinstance(hidden, torch.Tensor) or hidden.dim() != 2 or hidden.dtype != torch.int8 or not hidden.is_cuda:
        raise ValueError("hidden must be an int8 2-D device tensor")
    M, d = hidden.shape
    weight, V, packed = _head_arg(weight, d, "weight")
    if tokens.dim() != 2 or tokens.dtype != torch.int32:
        raise ValueError("tokens must be int32 [B, k]")
    B, k = tokens.shape
    dev = hidden.device
    if M != B * (k + 1):
        raise ValueError("hidden must hold B*(k+1) rows")
    if hidden_scale.shape != (M,) or weight_scale.shape != (V,) or hidden_scale.dtype != torch.float32 \
            or weight_scale.dtype != torch.float32:
        raise ValueError("hidden_scale [B*(k+1)] and weight_scale [V] must be float32")
    for t in (hidden, hidden_scale, weight, weight_scale, tokens):
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                           torch.empty((B, k + 1), dtype=torch.float32, device=dev), None, None)
    else:
        _check_out(out, B, k, dev, False)
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = int(lib().spec_lmhead_workspace_size(B, k, V, d))
    if need == 0:
        raise SpecVerifyError(-2, f"unsupported sizes B={B} k={k} V={V} d={d}")
    ws = _workspace(dev, stream, need) if workspace is None else _user_workspace(workspace, dev, need)
    args = (_ptr(hidden), _ptr(hidden_scale), _ptr(weight), _ptr(weight_scale), _ptr(tokens), B, k, V, d,
            _ptr(out.accepted_len), _ptr(out.out_tokens), _ptr(out.gap),
            ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), ctypes.c_void_p(stream))
    if phase_events is not None:
        if len(phase_events) != 3:
            raise ValueError("phase_events must hold three events")
        handles = []
        for ev in phase_events:
            if not ev.cuda_event:                         # torch creates events lazily
                ev.record(torch.cuda.current_stream(dev))
            handles.append(ev.cuda_event)
        arr = (ctypes.c_void_p * 3)(*handles)
        evp = ctypes.cast(arr, ctypes.c_void_p)
        rc = lib().spec_verify_lmhead_packed(*args, evp) if packed else lib().spec_verify_lmhead_timed(*args, evp)
    elif packed:
        rc = lib().spec_verify_lmhead_packed(*args, None)
    else:
        rc = lib().spec_verify_lmhead(*args)
    if rc != 0:
        raise SpecVerifyError(rc, last_error())
    return out


def spec_verify_lmhead_sample(hidden: torch.Tensor, hidden_scale: torch.Tensor, weight: torch.Tensor,
                              weight_scale: torch.Tensor, draft_hidden: Optional[torch.Tensor],
                              draft_hidden_scale: Optional[torch.Tensor], tokens: torch.Tensor,
                              uniforms: torch.Tensor, temperature: float, *,
                              draft_weight: Optional[torch.Tensor] = None,
                              draft_weight_scale: Optional[torch.Tensor] = None, return_probs: bool = True,
                              workspace: Optional[torch.Tensor] = None, out: Optional[VerifyResult] = None,
                              phase_events=None) -> VerifyResult:
    """Sampling-mode verification fused with int8 LM heads (see include/spec_verify.h).

    hidden int8 [B*(k+1), d] and hidden_scale float32 [B*(k+1)]: the target's
    rows (row b*(k+1)+i: position i of batch row b); draft_hidden int8 [B*k, d]
    and draft_hidden_scale [B*k] (None when k = 0); weight int8 [V, d] and
    weight_scale float32 [V]: the target's head, which the draft shares unless
    draft_weight / draft_weight_scale are given; tokens int32 [B, k]; uniforms
    float32 [B, k+1, 2]. weight and draft_weight may instead be PackedHead
    (pack_lmhead), both or neither. With phase_events (four torch.cuda.Event created with
    enable_timing=True) the call records them before the head passes, after
    them, after the merges of their records, and after the decisions and the
    draw.
    """
    if tokens.dim() != 2 or tokens.dtype != torch.int32:
        raise ValueError("tokens must be int32 [B, k]")
    B, k = tokens.shape
    if not isinstance(hidden, torch.Tensor) or hidden.dim() != 2 or hidden.dtype != torch.int8 or not hidden.is_cuda:
        raise ValueError("hidden must be an int8 2-D device tensor")
    M, d = hidden.shape
    weight, V, packed = _head_arg(weight, d, "weight")
    dev = hidden.device
    if M != B * (k + 1):
        raise ValueError("hidden must hold B*(k+1) rows")
    if hidden_scale.shape != (M,) or weight_scale.shape != (V,) or hidden_scale.dtype != torch.float32 \
            or weight_scale.dtype != torch.float32:
        raise ValueError("hidden_scale [B*(k+1)] and weight_scale [V] must be float32")
    if k > 0:
        if draft_hidden is None or draft_hidden_scale is None:
            raise ValueError("draft_hidden and draft_hidden_scale are required when k > 0")
        if draft_hidden.dtype != torch.int8 or tuple(draft_hidden.shape) != (B * k, d):
            raise ValueError("draft_hidden must be int8 [B*k, d]")
        if draft_hidden_scale.dtype != torch.float32 or tuple(draft_hidden_scale.shape) != (B * k,):
            raise ValueError("draft_hidden_scale must be float32 [B*k]")
    else:
        draft_hidden = draft_hidden_scale = None
    if (draft_weight is None) != (draft_weight_scale is None):
        raise ValueError("give draft_weight and draft_weight_scale together, or neither")
    if draft_weight is not None:
        draft_weight, dV, dpacked = _head_arg(draft_weight, d, "draft_weight")
        if dV != V or dpacked != packed:
            raise ValueError("draft_weight must be int8 [V, d], packed if and only if weight is")
        if draft_weight_scale.dtype != torch.float32 or tuple(draft_weight_scale.shape) != (V,):
            raise ValueError("draft_weight_scale must be float32 [V]")
    if uniforms.dtype != torch.float32 or tuple(uniforms.shape) != (B, k + 1, 2):
        raise ValueError("uniforms must be float32 [B, k+1, 2]")
    for t in (hidden, hidden_scale, weight, weight_scale, tokens, uniforms, draft_hidden, draft_hidden_scale,
              draft_weight, draft_weight_scale):
        if t is None:
            continue
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    probs = return_probs and k > 0
    if out is None:
        out = VerifyResult(torch.empty(B, dtype=torch.int32, device=dev),
                           torch.empty((B, k + 1), dtype=torch.int32, device=dev),
                           torch.empty((B, k + 1), dtype=torch.float32, device=dev),
                           torch.empty((B, k), dtype=torch.float32, device=dev) if probs else None,
                           torch.empty((B, k), dtype=torch.float32, device=dev) if probs else None)
    else:
        _check_out(out, B, k, dev, probs)
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = int(lib().spec_lmhead_sample_workspace_size(B, k, V, d))
    if need == 0:
        raise SpecVerifyError(-2, f"unsupported sizes B={B} k={k} V={V} d={d}")
    ws = _workspace(dev, stream, need) if workspace is None else _user_workspace(workspace, dev, need)
    args = (_ptr(hidden), _ptr(hidden_scale), _ptr(weight), _ptr(weight_scale), _ptr(draft_hidden),
            _ptr(draft_hidden_scale), _ptr(draft_weight), _ptr(draft_weight_scale), _ptr(tokens), _ptr(uniforms),
            float(temperature), B, k, V, d, _ptr(out.accepted_len), _ptr(out.out_tokens), _ptr(out.gap),
            _ptr(out.target_prob), _ptr(out.draft_prob),
            ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(), ctypes.c_void_p(stream))
    if phase_events is not None:
        if len(phase_events) != 4:
            raise ValueError("phase_events must hold four events")
        handles = []
        for ev in phase_events:
            if not ev.cuda_event:                         # torch creates events lazily
                ev.record(torch.cuda.current_stream(dev))
            handles.append(ev.cuda_event)
        arr = (ctypes.c_void_p * 4)(*handles)
        evp = ctypes.cast(arr, ctypes.c_void_p)
        rc = (lib().spec_verify_lmhead_sample_packed(*args, evp) if packed
              else lib().spec_verify_lmhead_sample_timed(*args, evp))
    elif packed:
        rc = lib().spec_verify_lmhead_sample_packed(*args, None)
    else:
        rc = lib().spec_verify_lmhead_sample(*args)
    if rc != 0:
        raise SpecVerifyError(rc, last_error())
    return out
