"""Batched speculative-decoding verification on AMD MI355X (gfx950).

Thin Python binding of libspecverify.so: every function has the name of the
C entry point it calls and only marshals arguments (torch tensors in device
memory, the current HIP stream, a zero-filled workspace).  All verification
work runs in the library's HIP kernels; there is no fallback: if the library
is missing or a call fails, an exception is raised.

    spec_workspace_bytes(B, n_pos, V)
    spec_fill_uniforms(seed, counter0, n, out=None)
    spec_verify_greedy(target, draft_tokens)
    spec_verify_sample(target, draft, draft_tokens, temperature, ...)
    spec_verify_sample_noalloc(target, draft, draft_tokens, temperature, ...)
    spec_verify_tree_greedy(target, parent, node_tokens)
    spec_verify_tree_sample(target, draft, parent, node_tokens, temperature, ...)
    spec_tree_depth(parent)
    spec_workspace_status(workspace), spec_workspace_reset(workspace)
"""
from __future__ import annotations

import ctypes
import functools
import os
import re
from typing import Optional, Sequence

import torch

__all__ = [
    "SpecVerifyError", "Workspace", "library_path", "load_library", "declared_symbols",
    "spec_workspace_bytes", "spec_fill_uniforms", "spec_verify_greedy",
    "spec_verify_sample", "spec_verify_sample_noalloc", "spec_verify_tree_greedy",
    "spec_verify_tree_sample", "spec_tree_depth", "spec_strerror",
    "spec_profile_enable", "spec_profile_read", "spec_profile_durations", "KERNEL_KINDS",
    "SCHEDULES",
    "spec_rejected_mask", "spec_tree_rejected_mask", "spec_tree_from_choices",
    "spec_workspace_status", "spec_workspace_reset", "STATUS_WAIT_GAVE_UP",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "spec_verify.h")

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_LOGITS, SPEC_PROBS = 0, 1
# spec_verify_sample schedules (SPEC_SCHED_*) and the test-only flag
SCHEDULES = {"auto": 0, "one_launch": 1, "two_launch": 2, "early_exit": 3}
SPEC_FLAG_TEST_GIVE_UP = 0x100
STATUS_WAIT_GAVE_UP = 1
SPEC_ESCRATCH = -6
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # SPEC_NOALLOC_SCRATCH_BYTES

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


def library_path() -> str:
    """The in-tree library, or the one SPEC_VERIFY_LIBRARY names (the
    host-sanitized build of the CPU tests)."""
    return os.environ.get("SPEC_VERIFY_LIBRARY") or os.path.join(_PKG, "libspecverify.so")


def declared_symbols() -> list:
    """Names of the functions declared in include/spec_verify.h."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def load_library():
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          f"or python -m verify_accept_sampling_amd._build")
    lib = ctypes.CDLL(path)
    c_int, c_size, c_u64, c_i64, c_f, vp = (ctypes.c_int, ctypes.c_size_t, ctypes.c_uint64,
                                            ctypes.c_int64, ctypes.c_float, ctypes.c_void_p)
    lib.spec_strerror.argtypes = [c_int]
    lib.spec_strerror.restype = ctypes.c_char_p
    lib.spec_workspace_bytes.argtypes = [c_int, c_int, c_int]
    lib.spec_workspace_bytes.restype = c_size
    lib.spec_fill_uniforms.argtypes = [c_u64, c_u64, c_i64, vp, vp]
    lib.spec_fill_uniforms.restype = c_int
    lib.spec_tree_depth.argtypes = [vp, c_int]
    lib.spec_tree_depth.restype = c_int
    lib.spec_verify_greedy.argtypes = [vp, c_int, c_int, c_int, c_int, vp, vp, vp, vp, c_size, vp]
    lib.spec_verify_greedy.restype = c_int
    lib.spec_verify_sample.argtypes = [vp, vp, c_int, c_int, c_int, c_int, c_int, vp, vp, c_u64,
                                       c_u64, c_f, c_int, vp, vp, vp, vp, c_size, vp]
    lib.spec_verify_sample.restype = c_int
    lib.spec_verify_sample_noalloc.argtypes = [vp, vp, c_int, c_int, c_int, c_int, c_int, vp, vp,
                                               c_u64, c_u64, c_f, c_int, vp, vp, vp, vp]
    lib.spec_verify_sample_noalloc.restype = c_int
    lib.spec_verify_tree_greedy.argtypes = [vp, c_int, c_int, c_int, c_int, vp, vp, vp, vp, vp,
                                            vp, c_size, vp]
    lib.spec_verify_tree_greedy.restype = c_int
    lib.spec_verify_tree_sample.argtypes = [vp, vp, c_int, c_int, c_int, c_int, c_int, vp, vp,
                                            vp, c_u64, c_u64, c_f, vp, vp, vp, vp, c_size, vp]
    lib.spec_verify_tree_sample.restype = c_int
    lib.spec_profile_enable.argtypes = [c_int]
    lib.spec_profile_enable.restype = c_int
    lib.spec_profile_read.argtypes = [c_int, ctypes.POINTER(ctypes.c_long),
                                      ctypes.POINTER(ctypes.c_double)]
    lib.spec_profile_read.restype = c_int
    lib.spec_profile_durations.argtypes = [c_int, ctypes.POINTER(ctypes.c_float), ctypes.c_long,
                                           ctypes.POINTER(ctypes.c_long)]
    lib.spec_profile_durations.restype = c_int
    lib.spec_workspace_status.argtypes = [vp, c_size, ctypes.POINTER(ctypes.c_uint32), vp]
    lib.spec_workspace_status.restype = c_int
    lib.spec_workspace_reset.argtypes = [vp, c_size, vp]
    lib.spec_workspace_reset.restype = c_int
    lib.spec_rejected_mask.argtypes = [vp, c_int, c_int, vp, vp, c_i64, vp]
    lib.spec_rejected_mask.restype = c_int
    lib.spec_tree_rejected_mask.argtypes = [vp, c_int, c_int, c_int, vp, vp, c_i64, vp]
    lib.spec_tree_rejected_mask.restype = c_int
    lib.spec_tree_from_choices.argtypes = [vp, vp, c_int, c_int, vp]
    lib.spec_tree_from_choices.restype = c_int
    _lib = lib
    return lib


KERNEL_KINDS = {"row_pass": 0, "draw": 1, "uniforms": 2, "fused": 3, "serving": 4,
                "tree_stats": 5, "tree_mass": 6, "tree_walk": 7, "tree_draw": 8,
                "tree_leaf": 9}


def spec_profile_enable(on: bool = True) -> None:
    """Start (clearing the totals) or stop per-kernel event timing."""
    _check(load_library().spec_profile_enable(1 if on else 0))


def spec_profile_read(kind: str):
    """(launches, total milliseconds) of one kernel kind since enabling."""
    n = ctypes.c_long(0)
    ms = ctypes.c_double(0.0)
    _check(load_library().spec_profile_read(KERNEL_KINDS[kind], ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def spec_profile_durations(kind: str) -> list:
    """Each timed launch's duration (ms, in launch order) of one kernel kind
    since enabling."""
    lib = load_library()
    n = ctypes.c_long(0)
    _check(lib.spec_profile_durations(KERNEL_KINDS[kind], None, 0, ctypes.byref(n)))
    buf = (ctypes.c_float * max(1, n.value))()
    _check(lib.spec_profile_durations(KERNEL_KINDS[kind], buf, n.value, ctypes.byref(n)))
    return [float(buf[i]) for i in range(n.value)]


def spec_strerror(code: int) -> str:
    return load_library().spec_strerror(int(code)).decode()


def _check(code: int):
    if code != 0:
        raise SpecVerifyError(code, spec_strerror(code))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> ctypes.c_void_p:
    # The raw handle of the current stream, without building a Stream object.
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _need_cuda(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@functools.lru_cache(maxsize=256)
def spec_workspace_bytes(B: int, n_pos: int, V: int) -> int:
    return int(load_library().spec_workspace_bytes(int(B), int(n_pos), int(V)))


class Workspace:
    """Zero-filled device workspace, grown on demand (zeroed again on growth).

    Calls leave its completion counters at zero, so it needs no clearing
    between calls of any shape.  Calls that share a workspace must be ordered
    on one stream; the default workspaces are one per (device, stream).  A
    buffer replaced on growth is released on the stream that allocated it
    (torch's caching allocator orders its reuse on that stream)."""

    def __init__(self, device=None):
        self.device = torch.device(device if device is not None else "cuda")
        self.buf = torch.zeros(0, dtype=torch.uint8, device=self.device)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 2 * self.buf.numel()), dtype=torch.uint8,
                                   device=self.device)
        return self.buf

    def status(self) -> int:
        """The workspace status word (waits for the current stream)."""
        return spec_workspace_status(self)

    def reset(self) -> None:
        """Zero the counter region on the current stream (after a failure)."""
        spec_workspace_reset(self)


_default_ws = {}


def _default_workspace(device) -> Workspace:
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, _stream(torch.device("cuda", idx)).value)
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(torch.device("cuda", idx))
    return ws


def _workspace(ws: Optional[Workspace], device, nbytes: int) -> torch.Tensor:
    if ws is None:
        ws = _default_workspace(device)
    return ws.get(nbytes)


def spec_workspace_status(workspace: Optional[Workspace] = None, device="cuda") -> int:
    """Status word of a workspace (0: no bounded wait gave up since the last
    reset; STATUS_WAIT_GAVE_UP otherwise).  Waits for the current stream."""
    ws = workspace if workspace is not None else _default_workspace(device)
    buf = ws.get(spec_workspace_bytes(0, 1, 1))  # at least the counter region
    v = ctypes.c_uint32(0)
    _check(load_library().spec_workspace_status(_ptr(buf), buf.numel(), ctypes.byref(v),
                                                _stream(buf.device)))
    return int(v.value)


def spec_workspace_reset(workspace: Optional[Workspace] = None, device="cuda") -> None:
    """Zero the counter region of a workspace (per-request words and status)
    on the current stream, so a workspace whose status is set can be used
    again."""
    ws = workspace if workspace is not None else _default_workspace(device)
    buf = ws.get(spec_workspace_bytes(0, 1, 1))  # at least the counter region
    _check(load_library().spec_workspace_reset(_ptr(buf), buf.numel(), _stream(buf.device)))


def spec_fill_uniforms(seed: int, counter0: int, n: int,
                       out: Optional[torch.Tensor] = None, device="cuda") -> torch.Tensor:
    if out is None:
        out = torch.empty(int(n), dtype=torch.float32, device=device)
    _need_cuda(out, "out")
    if out.dtype != torch.float32 or out.numel() < n:
        raise ValueError("out must be float32 with at least n elements")
    lib = load_library()
    _check(lib.spec_fill_uniforms(int(seed) & (2 ** 64 - 1), int(counter0) & (2 ** 64 - 1),
                                  int(n), _ptr(out), _stream(out.device)))
    return out


def spec_verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor,
                       workspace: Optional[Workspace] = None, out=None):
    """Greedy chain verification.  target [B, k+1, V] (f32/bf16), draft_tokens
    int32 [B, k].  out: optional preallocated (accepted_len, out_tokens),
    written in place and returned.  Returns (accepted_len [B], out_tokens
    [B, k+1])."""
    _need_cuda(target, "target")
    B, kp1, V = target.shape
    k = kp1 - 1
    _need_cuda(draft_tokens, "draft_tokens")
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, k):
        raise ValueError("draft_tokens must be int32 [B, k]")
    o_acc, o_out = (None, None) if out is None else out
    acc = _out_arg(o_acc, (B,), torch.int32, target.device, "accepted_len")
    out = _out_arg(o_out, (B, kp1), torch.int32, target.device, "out_tokens")
    lib = load_library()
    nbytes = spec_workspace_bytes(B, kp1, V)
    ws = _workspace(workspace, target.device, nbytes)
    _check(lib.spec_verify_greedy(_ptr(target), _dtype_code(target), B, k, V, _ptr(draft_tokens),
                                  _ptr(acc), _ptr(out), _ptr(ws), ws.numel(),
                                  _stream(target.device)))
    return acc, out


def _out_arg(t, shape, dtype, dev, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    _need_cuda(t, name)
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or t.device != dev:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         "on the inputs' device")
    return t


def _sample_args(target, draft, draft_tokens, uniforms, kind, schedule, out, probe,
                 test_give_up):
    """Checks and marshalling shared by both sampling entry points."""
    _need_cuda(target, "target")
    B, kp1, V = target.shape
    k = kp1 - 1
    dev = target.device
    if k > 0:
        _need_cuda(draft, "draft")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, k, V):
            raise ValueError("draft must match target's dtype with shape [B, k, V]")
        _need_cuda(draft_tokens, "draft_tokens")
        if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, k):
            raise ValueError("draft_tokens must be int32 [B, k]")
    if uniforms is not None:
        _need_cuda(uniforms, "uniforms")
        if uniforms.dtype != torch.float32 or uniforms.numel() != B * kp1 * 2:
            raise ValueError("uniforms must be float32 [B, k+1, 2]")
    kind_code = {"logits": SPEC_LOGITS, "probs": SPEC_PROBS}[kind]
    flags = SCHEDULES[schedule] | (SPEC_FLAG_TEST_GIVE_UP if test_give_up else 0)
    outs = tuple(out) if out is not None else (None, None, None)
    acc = _out_arg(outs[0], (B,), torch.int32, dev, "accepted_len")
    tok = _out_arg(outs[1], (B, kp1), torch.int32, dev, "out_tokens")
    pr = (_out_arg(outs[2] if len(outs) > 2 else None, (B, kp1, 4), torch.float32, dev, "probe")
          if probe else None)
    return B, k, V, dev, kind_code, flags, acc, tok, pr


def spec_verify_sample(target: torch.Tensor, draft: Optional[torch.Tensor],
                       draft_tokens: torch.Tensor, temperature: float = 1.0,
                       uniforms: Optional[torch.Tensor] = None, seed: int = 0,
                       counter0: int = 0, kind: str = "logits", probe: bool = False,
                       workspace: Optional[Workspace] = None, schedule: str = "auto",
                       out=None, test_give_up: bool = False):
    """Sampling chain verification with min(1, p/q) acceptance.

    target [B, k+1, V], draft [B, k, V] (f32/bf16 logits, or f32 probabilities
    with kind="probs"), draft_tokens int32 [B, k], uniforms float32
    [B, k+1, 2] or None (then derived from seed/counter0 inside the kernels).
    schedule: "auto", "one_launch", "two_launch" or "early_exit" (identical
    outputs).  out: optional preallocated (accepted_len, out_tokens[, probe])
    tensors, written in place and returned.  test_give_up: test only (see
    SPEC_FLAG_TEST_GIVE_UP in the C header).
    Returns (accepted_len, out_tokens) or, with probe=True,
    (accepted_len, out_tokens, probe [B, k+1, 4])."""
    B, k, V, dev, kind_code, flags, acc, tok, pr = _sample_args(
        target, draft, draft_tokens, uniforms, kind, schedule, out, probe, test_give_up)
    lib = load_library()
    nbytes = spec_workspace_bytes(B, k + 1, V)
    ws = _workspace(workspace, dev, nbytes)
    _check(lib.spec_verify_sample(
        _ptr(target), _ptr(draft if k > 0 else None), _dtype_code(target), kind_code, B, k, V,
        _ptr(draft_tokens if k > 0 else None), _ptr(uniforms),
        int(seed) & (2 ** 64 - 1), int(counter0) & (2 ** 64 - 1), float(temperature), flags,
        _ptr(acc), _ptr(tok), _ptr(pr), _ptr(ws), ws.numel(), _stream(dev)))
    if probe:
        return acc, tok, pr
    return acc, tok


def spec_verify_sample_noalloc(target: torch.Tensor, draft: Optional[torch.Tensor],
                               draft_tokens: torch.Tensor, temperature: float = 1.0,
                               uniforms: Optional[torch.Tensor] = None, seed: int = 0,
                               counter0: int = 0, kind: str = "logits", probe: bool = False,
                               schedule: str = "auto", out=None, test_give_up: bool = False):
    """spec_verify_sample on the library's static per-GPU scratch array (no
    workspace; the C call allocates nothing; pass `out` to allocate nothing
    here either).  Calls that overlap on one GPU race.  Raises
    SpecVerifyError (SPEC_ESCRATCH) for shapes beyond NOALLOC_SCRATCH_BYTES."""
    B, k, V, dev, kind_code, flags, acc, tok, pr = _sample_args(
        target, draft, draft_tokens, uniforms, kind, schedule, out, probe, test_give_up)
    lib = load_library()
    if dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError("spec_verify_sample_noalloc: the inputs must be on the current device")
    _check(lib.spec_verify_sample_noalloc(
        _ptr(target), _ptr(draft if k > 0 else None), _dtype_code(target), kind_code, B, k, V,
        _ptr(draft_tokens if k > 0 else None), _ptr(uniforms),
        int(seed) & (2 ** 64 - 1), int(counter0) & (2 ** 64 - 1), float(temperature), flags,
        _ptr(acc), _ptr(tok), _ptr(pr), _stream(dev)))
    if probe:
        return acc, tok, pr
    return acc, tok


_parent_cache: dict = {}


def _parent_array(parent) -> "ctypes.Array":
    """The parent array as int32 for the C call; the last few trees seen are
    kept (a deployment verifies against one static tree), so a repeated tree
    costs a tuple and a lookup."""
    key = tuple(parent.tolist() if hasattr(parent, "tolist") else parent)
    hit = _parent_cache.get(key)
    if hit is None:
        vals = [int(v) for v in key]
        hit = ((ctypes.c_int32 * len(vals))(*vals), len(vals))
        if len(_parent_cache) >= 8:
            _parent_cache.pop(next(iter(_parent_cache)))
        _parent_cache[key] = hit
    return hit


def spec_tree_depth(parent: Sequence[int]) -> int:
    arr, n = _parent_array(parent)
    d = int(load_library().spec_tree_depth(ctypes.cast(arr, ctypes.c_void_p), n))
    if d < 0:
        _check(d)
    return d


def spec_verify_tree_greedy(target: torch.Tensor, parent: Sequence[int],
                            node_tokens: torch.Tensor, want_path: bool = True,
                            workspace: Optional[Workspace] = None, out=None):
    """Greedy tree verification.  target [B, N, V], parent (host sequence of
    N ints), node_tokens int32 [B, N].  out: optional preallocated
    (accepted_len, out_tokens[, out_path]), written in place and returned.
    Returns (accepted_len [B], out_tokens [B, D+1], out_path [B, D+1] or
    None)."""
    _need_cuda(target, "target")
    B, N, V = target.shape
    _need_cuda(node_tokens, "node_tokens")
    if node_tokens.dtype != torch.int32 or tuple(node_tokens.shape) != (B, N):
        raise ValueError("node_tokens must be int32 [B, N]")
    arr, n = _parent_array(parent)
    if n != N:
        raise ValueError("parent must have one entry per node")
    D = int(load_library().spec_tree_depth(ctypes.cast(arr, ctypes.c_void_p), n))
    if D < 0:
        _check(D)
    dev = target.device
    outs = tuple(out) if out is not None else ()
    acc = _out_arg(outs[0] if outs else None, (B,), torch.int32, dev, "accepted_len")
    out = _out_arg(outs[1] if outs else None, (B, D + 1), torch.int32, dev, "out_tokens")
    if len(outs) > 2 and outs[2] is not None:
        path = _out_arg(outs[2], (B, D + 1), torch.int32, dev, "out_path")
    else:
        path = torch.empty(B, D + 1, dtype=torch.int32, device=dev) if want_path else None
    lib = load_library()
    nbytes = spec_workspace_bytes(B, N, V)
    ws = _workspace(workspace, dev, nbytes)
    _check(lib.spec_verify_tree_greedy(_ptr(target), _dtype_code(target), B, N, V,
                                       ctypes.cast(arr, ctypes.c_void_p), _ptr(node_tokens),
                                       _ptr(acc), _ptr(out), _ptr(path), _ptr(ws), ws.numel(),
                                       _stream(dev)))
    return acc, out, path


def spec_verify_tree_sample(target: torch.Tensor, draft: Optional[torch.Tensor],
                            parent: Sequence[int], node_tokens: torch.Tensor,
                            temperature: float = 1.0, uniforms: Optional[torch.Tensor] = None,
                            seed: int = 0, counter0: int = 0, kind: str = "logits",
                            want_path: bool = True, workspace: Optional[Workspace] = None,
                            out=None):
    """Sampling verification over a draft tree (siblings tried in index
    order, residual carried between them).  target, draft [B, N, V] (draft
    row j: the distribution node j's children were drawn from), parent (host
    sequence of N ints), node_tokens int32 [B, N], uniforms float32
    [B, N, 2] or None (seed/counter0).  out: optional preallocated
    (accepted_len, out_tokens[, out_path]).  Returns (accepted_len [B],
    out_tokens [B, D+1], out_path [B, D+1] or None)."""
    _need_cuda(target, "target")
    B, N, V = target.shape
    dev = target.device
    if N > 1:
        _need_cuda(draft, "draft")
        if draft.dtype != target.dtype or tuple(draft.shape) != (B, N, V):
            raise ValueError("draft must match target's dtype and shape [B, N, V]")
    _need_cuda(node_tokens, "node_tokens")
    if node_tokens.dtype != torch.int32 or tuple(node_tokens.shape) != (B, N):
        raise ValueError("node_tokens must be int32 [B, N]")
    if uniforms is not None:
        _need_cuda(uniforms, "uniforms")
        if uniforms.dtype != torch.float32 or uniforms.numel() != B * N * 2:
            raise ValueError("uniforms must be float32 [B, N, 2]")
    arr, n = _parent_array(parent)
    if n != N:
        raise ValueError("parent must have one entry per node")
    lib = load_library()
    D = int(lib.spec_tree_depth(ctypes.cast(arr, ctypes.c_void_p), n))
    if D < 0:
        _check(D)
    outs = tuple(out) if out is not None else (None, None, None)
    acc = _out_arg(outs[0], (B,), torch.int32, dev, "accepted_len")
    tok = _out_arg(outs[1], (B, D + 1), torch.int32, dev, "out_tokens")
    path = (_out_arg(outs[2] if len(outs) > 2 else None, (B, D + 1), torch.int32, dev,
                     "out_path") if want_path else None)
    kind_code = {"logits": SPEC_LOGITS, "probs": SPEC_PROBS}[kind]
    nbytes = spec_workspace_bytes(B, N, V)
    ws = _workspace(workspace, dev, nbytes)
    _check(lib.spec_verify_tree_sample(
        _ptr(target), _ptr(draft if N > 1 else None), _dtype_code(target), kind_code, B, N, V,
        ctypes.cast(arr, ctypes.c_void_p), _ptr(node_tokens), _ptr(uniforms),
        int(seed) & (2 ** 64 - 1), int(counter0) & (2 ** 64 - 1), float(temperature),
        _ptr(acc), _ptr(tok), _ptr(path), _ptr(ws), ws.numel(), _stream(dev)))
    return acc, tok, path


def _slot_arg(slot_mapping: Optional[torch.Tensor], shape, device) -> Optional[torch.Tensor]:
    if slot_mapping is None:
        return None
    _need_cuda(slot_mapping, "slot_mapping")
    if (slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != tuple(shape)
            or not slot_mapping.is_contiguous() or slot_mapping.device != device):
        raise ValueError(f"slot_mapping must be a contiguous int64 tensor of shape {tuple(shape)}"
                         " on the outputs' device")
    return slot_mapping


def spec_rejected_mask(accepted_len: torch.Tensor, k: int,
                       slot_mapping: Optional[torch.Tensor] = None, pad_slot: int = -1):
    """Rejected drafts of a chain verification: bool [B, k], True where
    i >= accepted_len[b].  With slot_mapping (int64 [B, k]), the rejected
    entries are set to pad_slot in place."""
    _need_cuda(accepted_len, "accepted_len")
    if accepted_len.dtype != torch.int32 or accepted_len.dim() != 1:
        raise ValueError("accepted_len must be int32 [B]")
    accepted_len = accepted_len.contiguous()
    B = accepted_len.shape[0]
    dev = accepted_len.device
    rej = torch.empty(B, k, dtype=torch.uint8, device=dev)
    slots = _slot_arg(slot_mapping, (B, k), dev)
    _check(load_library().spec_rejected_mask(_ptr(accepted_len), B, int(k), _ptr(rej),
                                             _ptr(slots), int(pad_slot), _stream(dev)))
    return rej.view(torch.bool)


def spec_tree_rejected_mask(out_path: torch.Tensor, n_nodes: int,
                            slot_mapping: Optional[torch.Tensor] = None, pad_slot: int = -1):
    """Rejected nodes of a tree verification: bool [B, n_nodes], True for
    every node j > 0 not on the accepted path out_path [B, D+1] (as
    returned by spec_verify_tree_greedy).  With slot_mapping (int64
    [B, n_nodes]), the rejected entries are set to pad_slot in place."""
    _need_cuda(out_path, "out_path")
    if out_path.dtype != torch.int32 or out_path.dim() != 2:
        raise ValueError("out_path must be int32 [B, D+1]")
    out_path = out_path.contiguous()
    B, D1 = out_path.shape
    dev = out_path.device
    rej = torch.empty(B, n_nodes, dtype=torch.uint8, device=dev)
    slots = _slot_arg(slot_mapping, (B, n_nodes), dev)
    _check(load_library().spec_tree_rejected_mask(_ptr(out_path), B, int(n_nodes), D1 - 1,
                                                  _ptr(rej), _ptr(slots), int(pad_slot),
                                                  _stream(dev)))
    return rej.view(torch.bool)


def spec_tree_from_choices(choices: Sequence[Sequence[int]]) -> list:
    """Parent array of a draft tree listed as choices (tuples of child ranks
    from the root, parents listed before children): node j+1 is choices[j],
    node 0 the root.  Host only."""
    seqs = [[int(v) for v in c] for c in choices]
    width = max([len(c) for c in seqs] + [1])
    flat = (ctypes.c_int32 * max(1, len(seqs) * width))()
    lens = (ctypes.c_int32 * max(1, len(seqs)))()
    for j, c in enumerate(seqs):
        lens[j] = len(c)
        for i, v in enumerate(c):
            flat[j * width + i] = v
    parent = (ctypes.c_int32 * (len(seqs) + 1))()
    rc = load_library().spec_tree_from_choices(ctypes.cast(flat, ctypes.c_void_p),
                                               ctypes.cast(lens, ctypes.c_void_p), len(seqs),
                                               width, ctypes.cast(parent, ctypes.c_void_p))
    if rc < 0:
        _check(rc)
    return list(parent)
