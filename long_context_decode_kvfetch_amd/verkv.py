"""Python binding of libverkv.so (the C ABI in include/verkv.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory, pinned host memory and streams.  If the
library is missing or cannot be loaded, importing the entry points raises; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# VERKV_LIBRARY names another build of the same sources (the host-sanitizer build)
LIB_PATH = os.environ.get("VERKV_LIBRARY") or os.path.join(_HERE, "libverkv.so")

OK, EINVAL, EBUDGET, ECAPACITY, EHIP, EUNSUPPORTED, EWORKSPACE = 0, -1, -2, -3, -4, -5, -6
BF16, F32 = 0, 1
HEAD_DIM = 128
PROFILE_KINDS = 14
KERNEL_NAMES = ["poissoncomp", "gather_pivots", "sketch_scores", "decide", "union_lists",
                "attend_pivots", "attend_host", "finish", "eps_after", "pivot_coef", "prefetch",
                "quantize_sketch", "resolve", "stage_plan"]


class VerKVError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        msg = f"{what}: {_lib().verkv_status_str(status).decode()} ({status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


class Shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_kv_heads", C.c_int32), ("group", C.c_int32),
                ("head_dim", C.c_int32), ("seq_len", C.POINTER(C.c_int32)),
                ("n_sink", C.c_int32), ("n_local", C.c_int32), ("kv_dtype", C.c_int32),
                ("layer", C.c_uint32), ("seq_cap", C.POINTER(C.c_int32)),
                ("stage_slots", C.c_int32)]


class State(C.Structure):
    _fields_ = [("r", C.c_void_p), ("resident", C.c_void_p), ("piv_idx", C.c_void_p),
                ("piv_count", C.c_void_p), ("piv_k", C.c_void_p), ("piv_v", C.c_void_p),
                ("cap", C.c_int32), ("sketch", C.c_void_p), ("sketch_exact", C.c_int32),
                ("v_host", C.c_void_p), ("sketch_format", C.c_int32), ("level", C.c_void_p),
                ("k_host", C.c_void_p)]


SKETCH_ROWS, SKETCH_2BIT, SKETCH2_ROW_BYTES = 0, 1, 64


class StepOut(C.Structure):
    _fields_ = [("m_hat", C.c_void_p), ("d_sketch", C.c_void_p), ("beta_star", C.c_void_p),
                ("eps_hat", C.c_void_p), ("certified", C.c_void_p), ("kstar", C.c_void_p),
                ("fetch_idx", C.c_void_p), ("fetch_cap", C.c_int32), ("fetch_count", C.c_void_p),
                ("h2d_count", C.c_void_p), ("eps_after", C.c_void_p), ("n_hat", C.c_void_p),
                ("d_hat", C.c_void_p), ("o", C.c_void_p), ("lse", C.c_void_p)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run long_context_decode_kvfetch_amd.build")
        lib = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        lib.verkv_status_str.restype = C.c_char_p
        lib.verkv_status_str.argtypes = [i32]
        lib.verkv_last_error.restype = C.c_char_p
        lib.verkv_version.restype = i32
        lib.verkv_source_hash.restype = C.c_char_p
        lib.verkv_compress_workspace_bytes.restype = sz
        lib.verkv_compress_workspace_bytes.argtypes = [C.POINTER(Shape)]
        lib.verkv_decode_workspace_bytes.restype = sz
        lib.verkv_decode_workspace_bytes.argtypes = [C.POINTER(Shape), i32]
        lib.verkv_staged_rows.restype = i32
        lib.verkv_staged_rows.argtypes = [vp, sz, C.POINTER(Shape), i32, vp, C.POINTER(C.c_int64)]
        lib.verkv_pivot_rows.restype = sz
        lib.verkv_pivot_rows.argtypes = [C.POINTER(Shape), i32]
        lib.verkv_quantize_sketch.restype = i32
        lib.verkv_quantize_sketch.argtypes = [C.POINTER(Shape), vp, vp, vp]
        lib.verkv_append.restype = i32
        lib.verkv_append.argtypes = [C.POINTER(Shape), C.POINTER(State), vp, vp, vp, C.c_uint64,
                                     vp, vp, sz, vp]
        lib.verkv_append_workspace_bytes.restype = sz
        lib.verkv_append_workspace_bytes.argtypes = [C.POINTER(Shape), i32]
        lib.verkv_compress.restype = i32
        lib.verkv_compress.argtypes = [C.POINTER(Shape), vp, vp, vp, C.c_double, C.c_uint64,
                                       C.POINTER(State), vp, sz, C.POINTER(i32), vp]
        lib.verkv_decode_step.restype = i32
        lib.verkv_decode_step.argtypes = [C.POINTER(Shape), C.POINTER(State), vp, C.c_double,
                                          C.c_double, C.c_double, C.POINTER(StepOut), vp, sz, vp]
        lib.verkv_decode_step_ex.restype = i32
        lib.verkv_decode_step_ex.argtypes = [C.POINTER(Shape), C.POINTER(State), vp, C.c_double,
                                             C.c_double, C.c_double, C.POINTER(StepOut), vp, sz,
                                             C.c_uint32, vp]
        lib.verkv_refine.restype = i32
        lib.verkv_refine.argtypes = [C.POINTER(Shape), C.POINTER(State), vp, vp, vp,
                                     C.POINTER(StepOut), vp, sz, vp]
        lib.verkv_profile_begin.restype = i32
        lib.verkv_profile_begin.argtypes = [i32]
        lib.verkv_profile_report.restype = i32
        lib.verkv_profile_report.argtypes = [C.POINTER(C.c_double), C.POINTER(i32), i32]
        lib.verkv_profile_end.restype = None
        lib.verkv_step_noalloc.restype = i32
        lib.verkv_step_noalloc.argtypes = [C.POINTER(Shape), C.POINTER(State), vp, C.c_double,
                                           C.c_double, C.c_double, vp, vp, C.POINTER(StepOut),
                                           vp, vp]
        lib.verkv_noalloc_scratch_bytes.restype = sz
        lib.verkv_gather_rows_memcpy.restype = i32
        lib.verkv_gather_rows_memcpy.argtypes = [vp, sz, vp, i32, vp, C.POINTER(C.c_int64), vp]
        lib.verkv_check.restype = i32
        lib.verkv_check.argtypes = [vp, C.POINTER(Shape), i32, vp]
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def built_from_current_sources() -> bool:
    """True if the loaded library carries the hash of the sources in this tree."""
    from . import build
    return _lib().verkv_source_hash().decode() == build.source_hash()


def _check(status: int, what: str):
    if status != OK:
        raise VerKVError(status, what, _lib().verkv_last_error().decode())


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ----------------------------------------------------------------------------- shapes
@dataclass
class LayerShape:
    """Shape of one layer of a (possibly ragged) batch."""
    seq_lens: list
    n_kv_heads: int
    group: int
    n_sink: int
    n_local: int
    kv_dtype: str = "bf16"
    layer: int = 0
    seq_caps: list | None = None     # token capacity per sequence (None: the lengths)
    stage_slots: int = 0             # cross-step staging rows per KV head (0: the default)

    def __post_init__(self):
        self._lens = (C.c_int32 * len(self.seq_lens))(*[int(x) for x in self.seq_lens])
        caps = self.seq_caps if self.seq_caps is not None else self.seq_lens
        self._caps = (C.c_int32 * len(caps))(*[int(x) for x in caps])
        self.c = Shape(len(self.seq_lens), self.n_kv_heads, self.group, HEAD_DIM,
                       C.cast(self._lens, C.POINTER(C.c_int32)), self.n_sink, self.n_local,
                       BF16 if self.kv_dtype == "bf16" else F32, self.layer,
                       C.cast(self._caps, C.POINTER(C.c_int32)), int(self.stage_slots))

    def grown(self, by: int = 1) -> "LayerShape":
        """The same layer after `by` tokens were appended to every sequence."""
        return LayerShape([n + by for n in self.seq_lens], self.n_kv_heads, self.group,
                          self.n_sink, self.n_local, self.kv_dtype, self.layer,
                          list(self.caps), self.stage_slots)

    @property
    def caps(self):
        return list(self.seq_caps) if self.seq_caps is not None else list(self.seq_lens)

    @property
    def total_slots(self):
        """Token slots of the capacity-strided arrays (sum of capacities)."""
        return int(sum(self.caps))

    @property
    def batch(self):
        return len(self.seq_lens)

    @property
    def n_q_heads(self):
        return self.n_kv_heads * self.group

    @property
    def total_tokens(self):
        return int(sum(self.seq_lens))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.kv_dtype == "bf16" else torch.float32

    def append_workspace_bytes(self, cap: int) -> int:
        return int(_lib().verkv_append_workspace_bytes(C.byref(self.c), int(cap)))

    def compress_workspace_bytes(self) -> int:
        return int(_lib().verkv_compress_workspace_bytes(C.byref(self.c)))

    def decode_workspace_bytes(self, cap: int) -> int:
        return int(_lib().verkv_decode_workspace_bytes(C.byref(self.c), int(cap)))

    def pivot_rows(self, cap: int) -> int:
        return int(_lib().verkv_pivot_rows(C.byref(self.c), int(cap)))


def default_cap(shape: LayerShape, eta: float) -> int:
    """A pivot capacity that holds H u S with overwhelming probability: the forced
    tokens plus eta*n_max plus 8 standard deviations, rounded up to 64."""
    n = max(shape.seq_lens)
    mean = eta * n
    cap = min(n, int(mean + 8.0 * math.sqrt(max(mean, 1.0)) + shape.n_sink + shape.n_local + 64))
    return ((cap + 63) // 64) * 64


# ----------------------------------------------------------------------------- buffers
class LayerState:
    """GPU-resident compressed state of one layer (caller-owned torch buffers)."""

    def __init__(self, shape: LayerShape, cap: int, sketch: torch.Tensor, device="cuda",
                 sketch_exact: bool = True, v_host: torch.Tensor | None = None,
                 sketch_format: int = SKETCH_ROWS, k_host: torch.Tensor | None = None):
        hkv, tot = shape.n_kv_heads, shape.total_slots
        words = sum((n + 31) // 32 for n in shape.caps)
        units = shape.batch * hkv
        self.shape = shape
        self.cap = int(cap)
        self.r = torch.empty(hkv * tot, dtype=torch.float64, device=device)
        self.resident = torch.empty(hkv * words, dtype=torch.int32, device=device)
        self.piv_idx = torch.empty(units * cap, dtype=torch.int32, device=device)
        self.piv_count = torch.empty(units, dtype=torch.int32, device=device)
        prow = shape.pivot_rows(cap)            # pivot K/V rows, stored in schedule order
        self.piv_k = torch.empty(prow * HEAD_DIM, dtype=shape.torch_dtype, device=device)
        self.piv_v = torch.empty(prow * HEAD_DIM, dtype=shape.torch_dtype, device=device)
        self.level = torch.empty(units, dtype=torch.float64, device=device)
        self.sketch = sketch
        self.v_host = v_host                    # kept alive with the state
        self.k_host = k_host
        self.c = State(_ptr(self.r), _ptr(self.resident), _ptr(self.piv_idx), _ptr(self.piv_count),
                       _ptr(self.piv_k), _ptr(self.piv_v), self.cap, _ptr(sketch),
                       1 if sketch_exact else 0, _ptr(v_host) if v_host is not None else None,
                       int(sketch_format), _ptr(self.level),
                       _ptr(k_host) if k_host is not None else None)


class StepBuffers:
    """Per-step outputs (caller-owned torch buffers)."""

    def __init__(self, shape: LayerShape, fetch_cap: int | None = None, device="cuda"):
        rows = shape.batch * shape.n_q_heads
        units = shape.batch * shape.n_kv_heads
        f64 = dict(dtype=torch.float64, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.m_hat = torch.empty(rows, **f64)
        self.d_sketch = torch.empty(rows, **f64)
        self.beta_star = torch.empty(rows, **f64)
        self.eps_hat = torch.empty(rows, **f64)
        self.certified = torch.empty(rows, dtype=torch.uint8, device=device)
        self.kstar = torch.empty(rows, **i32)
        self.fetch_cap = int(fetch_cap if fetch_cap is not None else max(shape.seq_lens))
        self.fetch_idx = torch.empty(units * self.fetch_cap, **i32) if self.fetch_cap > 0 else None
        self.fetch_count = torch.empty(units, **i32)
        self.h2d_count = torch.empty(units, **i32)
        self.eps_after = torch.empty(rows, **f64)
        self.n_hat = torch.empty(rows * HEAD_DIM, **f32)
        self.d_hat = torch.empty(rows, **f32)
        self.o = torch.empty(rows * HEAD_DIM, **f32)
        self.lse = torch.empty(rows, **f32)
        self.c = StepOut(_ptr(self.m_hat), _ptr(self.d_sketch), _ptr(self.beta_star),
                         _ptr(self.eps_hat), _ptr(self.certified), _ptr(self.kstar),
                         _ptr(self.fetch_idx), self.fetch_cap if self.fetch_idx is not None else 0,
                         _ptr(self.fetch_count), _ptr(self.h2d_count), _ptr(self.eps_after),
                         _ptr(self.n_hat), _ptr(self.d_hat), _ptr(self.o), _ptr(self.lse))

    def fetch_lists(self, shape: LayerShape):
        """Per (sequence, KV head) ascending fetch lists as numpy arrays (synchronises)."""
        cnt = self.fetch_count.cpu().numpy()
        idx = self.fetch_idx.view(-1, self.fetch_cap).cpu().numpy()
        return [idx[u, :min(int(cnt[u]), self.fetch_cap)] for u in range(cnt.size)]


# ----------------------------------------------------------------------------- entry points
def compress(shape: LayerShape, tau: torch.Tensor, K_host: torch.Tensor, V_host: torch.Tensor,
             eta: float, seed: int, state: LayerState, workspace: torch.Tensor, stream=None) -> int:
    """verkv_compress; returns the largest pivot count.  Raises VerKVError."""
    need = C.c_int32(0)
    st = _lib().verkv_compress(C.byref(shape.c), _ptr(tau), _ptr(K_host), _ptr(V_host),
                               float(eta), int(seed) & ((1 << 64) - 1), C.byref(state.c),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               C.byref(need), _stream(stream))
    if st == ECAPACITY:
        err = VerKVError(st, "verkv_compress", f"needed cap {need.value} > {state.cap}")
        err.needed_cap = need.value
        raise err
    _check(st, "verkv_compress")
    return need.value


def append(shape: LayerShape, state: LayerState, tau: torch.Tensor, K_host: torch.Tensor,
           V_host: torch.Tensor, seed: int, status: torch.Tensor, workspace: torch.Tensor,
           stream=None) -> None:
    """verkv_append: token n_b appended to every sequence (asynchronous on `stream`);
    `shape` has the lengths before the append, `status` is a 4-byte device word."""
    _check(_lib().verkv_append(C.byref(shape.c), C.byref(state.c), _ptr(tau), _ptr(K_host),
                               _ptr(V_host), int(seed) & ((1 << 64) - 1), _ptr(status),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream)),
           "verkv_append")


def quantize_sketch(shape: LayerShape, K: torch.Tensor, sketch: torch.Tensor, stream=None) -> None:
    """verkv_quantize_sketch: the 2-bit sketch rows of K (asynchronous on `stream`)."""
    need = shape.total_slots * shape.n_kv_heads * SKETCH2_ROW_BYTES
    if sketch.numel() * sketch.element_size() < need:
        raise ValueError(f"sketch buffer holds {sketch.numel() * sketch.element_size()} B, needs {need}")
    _check(_lib().verkv_quantize_sketch(C.byref(shape.c), _ptr(K), _ptr(sketch), _stream(stream)),
           "verkv_quantize_sketch")


STEP_RESOLVED = 1


def decode_step(shape: LayerShape, state: LayerState, q: torch.Tensor, beta: float, eps: float,
                delta: float, out: StepBuffers, workspace: torch.Tensor, stream=None,
                resolved: bool = False) -> None:
    """verkv_decode_step, or verkv_decode_step_ex with VERKV_STEP_RESOLVED (the bias
    re-solved on each candidate set of the k* cut); asynchronous on `stream`."""
    if resolved:
        _check(_lib().verkv_decode_step_ex(C.byref(shape.c), C.byref(state.c), _ptr(q),
                                           float(beta), float(eps), float(delta), C.byref(out.c),
                                           _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           STEP_RESOLVED, _stream(stream)),
               "verkv_decode_step_ex")
        return
    _check(_lib().verkv_decode_step(C.byref(shape.c), C.byref(state.c), _ptr(q), float(beta),
                                    float(eps), float(delta), C.byref(out.c), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)),
           "verkv_decode_step")


def refine(shape: LayerShape, state: LayerState, q: torch.Tensor, K_host: torch.Tensor,
           V_host: torch.Tensor, out: StepBuffers, workspace: torch.Tensor, stream=None) -> None:
    """verkv_refine (asynchronous on `stream`)."""
    _check(_lib().verkv_refine(C.byref(shape.c), C.byref(state.c), _ptr(q), _ptr(K_host),
                               _ptr(V_host), C.byref(out.c), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "verkv_refine")


def step_noalloc(shape: LayerShape, state: LayerState, q: torch.Tensor, beta: float, eps: float,
                 delta: float, K_host: torch.Tensor, V_host: torch.Tensor, out: StepBuffers,
                 status: torch.Tensor | None = None, stream=None) -> None:
    """verkv_step_noalloc: decode step and refinement on the library's static scratch
    (asynchronous on `stream`)."""
    _check(_lib().verkv_step_noalloc(C.byref(shape.c), C.byref(state.c), _ptr(q), float(beta),
                                     float(eps), float(delta), _ptr(K_host), _ptr(V_host),
                                     C.byref(out.c), _ptr(status), _stream(stream)),
           "verkv_step_noalloc")


def gather_rows_memcpy(src_ptr: int, row_bytes: int, idx, dst_ptr: int, stream=None) -> int:
    """verkv_gather_rows_memcpy: rows idx (ascending, host int32 array) of the row array
    at src_ptr to dst_ptr, one hipMemcpyAsync per run of consecutive rows (asynchronous
    on `stream`).  Returns the number of copies issued."""
    import numpy as np
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    runs = C.c_int64(0)
    _check(_lib().verkv_gather_rows_memcpy(C.c_void_p(src_ptr), int(row_bytes),
                                           idx.ctypes.data_as(C.c_void_p), int(idx.size),
                                           C.c_void_p(dst_ptr), C.byref(runs), _stream(stream)),
           "verkv_gather_rows_memcpy")
    return runs.value


def staged_rows(shape: LayerShape, cap: int, workspace: torch.Tensor, stream=None) -> int:
    """verkv_staged_rows: rows of the last refine on `workspace` taken from the staging area
    instead of the host link (synchronises `stream`)."""
    rows = C.c_int64(0)
    _check(_lib().verkv_staged_rows(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                    C.byref(shape.c), int(cap), _stream(stream), C.byref(rows)),
           "verkv_staged_rows")
    return int(rows.value)


def check(shape: LayerShape, cap: int, workspace: torch.Tensor, stream=None) -> None:
    """verkv_check: synchronise and raise if the kernels flagged a problem."""
    _check(_lib().verkv_check(_ptr(workspace), C.byref(shape.c), int(cap), _stream(stream)),
           "verkv_check")


def profile_begin(max_launches: int) -> None:
    _check(_lib().verkv_profile_begin(int(max_launches)), "verkv_profile_begin")


def profile_report():
    """{kernel name: (total_ms, launches)} of the launches recorded since the last report."""
    ms = (C.c_double * PROFILE_KINDS)()
    cnt = (C.c_int32 * PROFILE_KINDS)()
    _check(_lib().verkv_profile_report(ms, cnt, PROFILE_KINDS), "verkv_profile_report")
    return {KERNEL_NAMES[k]: (ms[k], cnt[k]) for k in range(PROFILE_KINDS)}


def profile_end() -> None:
    _lib().verkv_profile_end()


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
