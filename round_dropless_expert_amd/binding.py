"""ctypes binding of libmoe_rounds.so (the C ABI in include/moe_rounds.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. Device buffers are torch tensors (or raw device addresses); torch
provides device memory and the current stream, nothing else. If the library
has not been built this module raises at load time: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import torch  # loads the HIP runtime the library must share

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libmoe_rounds.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_F32 = 0
MOE_BF16 = 1

MOE_WEIGHTS_ROW_MAJOR = 0
MOE_WEIGHTS_TILED = 1

EXPORTS = ("moe_status_string", "moe_last_error", "moe_hip_runtime_version",
           "moe_check_config", "moe_workspace_size", "moe_forward_workspace_size",
           "moe_workspace_layout",
           "moe_plan", "moe_launch_batches", "moe_dispatch", "moe_expert_ffn",
           "moe_expert_gate_up",
           "moe_expert_down", "moe_dispatch_gate_up", "moe_pack_weights", "moe_combine", "moe_forward",
           "moe_capacity_curve", "moe_capacity_for_rounds",
           "moe_backward_workspace_size", "moe_backward_layout",
           "moe_backward", "moe_forward_static")


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("C", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("weight_layout", ctypes.c_int32),
                ("group", ctypes.c_int32), ("round_buffers", ctypes.c_int32)]


LAYOUT_FIELDS = ("idx", "weight", "counts", "offsets", "n_rounds", "perm",
                 "pos", "round_of", "row_of", "rounds", "scratch", "xr", "h",
                 "z")


class MoeLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in LAYOUT_FIELDS] + \
        [("total", ctypes.c_size_t)]


BWD_LAYOUT_FIELDS = ("xr", "dyr", "gu", "hw", "dgu", "dz", "ones")


class MoeBackwardLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in BWD_LAYOUT_FIELDS] + \
        [("total", ctypes.c_size_t)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it is missing: no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python round_dropless_expert_amd/csrc/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i32p = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                         ctypes.POINTER(ctypes.c_int32))
    cfgp = ctypes.POINTER(MoeConfig)
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_hip_runtime_version.argtypes = []
    L.moe_hip_runtime_version.restype = ctypes.c_int32
    L.moe_check_config.argtypes = [cfgp]
    L.moe_workspace_size.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_forward_workspace_size.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_workspace_layout.argtypes = [cfgp, ctypes.POINTER(MoeLayout)]
    L.moe_plan.argtypes = [cfgp, vp, vp, sz, i32p, vp]
    L.moe_launch_batches.argtypes = [cfgp, i32p, i32, i32p, i32p, i32p]
    L.moe_dispatch.argtypes = [cfgp, i32, i32, vp, vp, sz, vp]
    L.moe_expert_ffn.argtypes = [cfgp, i32, i32, vp, vp, vp, i32p, vp, sz, vp]
    L.moe_expert_gate_up.argtypes = [cfgp, i32, i32, vp, vp, i32p, vp, sz, vp]
    L.moe_expert_down.argtypes = [cfgp, i32, i32, vp, i32p, vp, sz, vp]
    L.moe_dispatch_gate_up.argtypes = [cfgp, i32, i32, vp, vp, vp, i32p, vp, sz, vp]
    L.moe_pack_weights.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_combine.argtypes = [cfgp, vp, sz, vp, vp]
    L.moe_forward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward_static.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp]
    i64, i64p = ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)
    L.moe_capacity_curve.argtypes = [cfgp, i32p, i64, i64p, i32, i32p,
                                     ctypes.POINTER(ctypes.c_size_t)]
    L.moe_capacity_for_rounds.argtypes = [cfgp, i32p, i64, i32, ctypes.c_double,
                                          i64p]
    L.moe_backward_workspace_size.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_backward_layout.argtypes = [cfgp, ctypes.POINTER(MoeBackwardLayout)]
    L.moe_backward.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                               vp, sz, vp, sz, vp]
    for n in ("moe_check_config", "moe_workspace_size", "moe_forward_workspace_size",
              "moe_workspace_layout",
              "moe_plan", "moe_launch_batches", "moe_dispatch", "moe_expert_ffn",
              "moe_expert_gate_up", "moe_expert_down", "moe_dispatch_gate_up",
              "moe_pack_weights",
              "moe_combine", "moe_forward", "moe_capacity_curve",
              "moe_capacity_for_rounds", "moe_backward_workspace_size",
              "moe_backward_layout", "moe_backward",
              "moe_forward_static"):
        getattr(L, n).restype = ctypes.c_int
    _lib = L
    return L


def check_runtime() -> None:
    """The library must run on the same HIP runtime instance as torch."""
    v = load().moe_hip_runtime_version()
    want = torch.version.hip
    if want is None:
        raise RuntimeError("torch was built without HIP")
    major, minor = (int(x) for x in want.split(".")[:2])
    if v < 0 or v // 10_000_000 != major or (v // 100_000) % 100 != minor:
        raise RuntimeError(f"libmoe_rounds sees HIP runtime {v}, torch uses {want}")


def _check(status: int) -> None:
    if status != MOE_OK:
        L = load()
        raise MoeError(status, f"{L.moe_status_string(status).decode()}: "
                               f"{L.moe_last_error().decode()}")


def config(T, E, k, d_model, d_ff, C, dtype,
           weight_layout=MOE_WEIGHTS_ROW_MAJOR, group=1,
           round_buffers=1) -> MoeConfig:
    """group: experts per capacity group (1 = strict per-expert capacity);
    round_buffers: 1, or 2 to overlap consecutive rounds in moe_forward."""
    if isinstance(dtype, str):
        dtype = {"f32": MOE_F32, "bf16": MOE_BF16}[dtype]
    elif isinstance(dtype, torch.dtype):
        dtype = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}[dtype]
    if isinstance(weight_layout, str):
        weight_layout = {"row_major": MOE_WEIGHTS_ROW_MAJOR,
                         "tiled": MOE_WEIGHTS_TILED}[weight_layout]
    return MoeConfig(int(T), int(E), int(k), int(d_model), int(d_ff), int(C),
                     int(dtype), int(weight_layout), int(group),
                     int(round_buffers))


def buffer_geometry(cfg: MoeConfig) -> dict:
    """Round-buffer geometry: C' = min(C, T), P = C' rounded up to 64, the
    group size G, rows per group Q (P for G = 1, else G*(P+64)), the rows of
    one set of round buffers, the number of sets S (round r uses set r % S)
    and the rows M of each round table."""
    ce = min(cfg.C, cfg.T)
    pad = (ce + 63) // 64 * 64
    G = cfg.group if cfg.group > 0 else 1
    Q = pad if G == 1 else G * (pad + 64)
    S = cfg.round_buffers if cfg.round_buffers > 0 else 1
    return {"ce": ce, "pad": pad, "G": G, "Q": Q, "rows": (cfg.E // G) * Q,
            "S": S, "M": -(-cfg.T // ce)}


def check_config(cfg: MoeConfig) -> int:
    return load().moe_check_config(ctypes.byref(cfg))


def workspace_size(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def forward_workspace_size(cfg: MoeConfig) -> int:
    """Bytes moe_forward and moe_backward need (the workspace up to xr when
    the forward gathers its rows from x)."""
    n = ctypes.c_size_t(0)
    _check(load().moe_forward_workspace_size(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def workspace_layout(cfg: MoeConfig) -> dict:
    L = MoeLayout()
    _check(load().moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)))
    return {n: getattr(L, n) for n in LAYOUT_FIELDS + ("total",)}


def _ptr(t) -> int:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _arg(t, name, dtype=None, numel=None):
    """Device address of a tensor argument, after checking what the C ABI
    cannot see from a pointer: a device (cuda) tensor, contiguous, of the
    element type and with at least the elements the config implies. A host
    tensor would otherwise reach a kernel as a host address. None and raw
    integer addresses pass unchanged."""
    if t is None or isinstance(t, int):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor or an int address")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device (cuda) tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the config needs {numel}")
    return t.data_ptr()


def _el(cfg) -> "torch.dtype":
    return torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(ws) -> int:
    return ws.numel() * ws.element_size()


def moe_plan(cfg, logits, ws, read_rounds=True, stream=None,
             return_counts=False):
    """Route + plan. With read_rounds (waits for the stream) returns R, or
    (R, counts) with return_counts (counts: int32 numpy array of E, the
    counts_host argument of the expert calls)."""
    out = (ctypes.c_int32 * (cfg.E + 1))()
    _check(load().moe_plan(ctypes.byref(cfg),
                           _arg(logits, "logits", torch.float32, cfg.T * cfg.E),
                           _arg(ws, "ws"),
                           _nbytes(ws), out if read_rounds else None,
                           _stream(stream)))
    if not read_rounds:
        return None
    vals = np.frombuffer(out, dtype=np.int32).copy()
    return (int(vals[-1]), vals[:-1].copy()) if return_counts else int(vals[-1])


def _counts(counts_host):
    if counts_host is None:
        return None
    a = np.ascontiguousarray(counts_host, dtype=np.int32)
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), a


def launch_batches(cfg, counts_host):
    """The forward's launch batches for a step's counts: a list of
    (first_round, n_rounds)."""
    a = np.ascontiguousarray(counts_host, dtype=np.int32)
    n_max = max(1, -(-cfg.T // max(1, min(cfg.C, cfg.T))))
    first = np.zeros(n_max, dtype=np.int32)
    nr = np.zeros(n_max, dtype=np.int32)
    n = ctypes.c_int32(0)
    p32 = lambda v: v.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(load().moe_launch_batches(ctypes.byref(cfg), p32(a), n_max, p32(first),
                                     p32(nr), ctypes.byref(n)))
    return [(int(first[i]), int(nr[i])) for i in range(n.value)]


def moe_dispatch(cfg, round_, x, ws, stream=None, n_rounds=1):
    _check(load().moe_dispatch(ctypes.byref(cfg), int(round_), int(n_rounds),
                               _arg(x, "x", _el(cfg), cfg.T * cfg.d_model),
                               _arg(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_expert_ffn(cfg, round_, w_gate, w_up, w_down, ws, stream=None,
                   counts_host=None, n_rounds=1):
    c = _counts(counts_host)
    nw = cfg.E * cfg.d_model * cfg.d_ff
    _check(load().moe_expert_ffn(ctypes.byref(cfg), int(round_), int(n_rounds),
                                 _arg(w_gate, "w_gate", _el(cfg), nw),
                                 _arg(w_up, "w_up", _el(cfg), nw),
                                 _arg(w_down, "w_down", _el(cfg), nw), c and c[0],
                                 _arg(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_expert_gate_up(cfg, round_, w_gate, w_up, ws, stream=None,
                       counts_host=None, n_rounds=1):
    c = _counts(counts_host)
    nw = cfg.E * cfg.d_model * cfg.d_ff
    _check(load().moe_expert_gate_up(ctypes.byref(cfg), int(round_), int(n_rounds),
                                     _arg(w_gate, "w_gate", _el(cfg), nw),
                                     _arg(w_up, "w_up", _el(cfg), nw), c and c[0],
                                     _arg(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_dispatch_gate_up(cfg, round_, x, w_gate, w_up, ws, stream=None,
                         counts_host=None, n_rounds=1):
    c = _counts(counts_host)
    nw = cfg.E * cfg.d_model * cfg.d_ff
    _check(load().moe_dispatch_gate_up(ctypes.byref(cfg), int(round_), int(n_rounds),
                                       _arg(x, "x", _el(cfg), cfg.T * cfg.d_model),
                                       _arg(w_gate, "w_gate", _el(cfg), nw),
                                       _arg(w_up, "w_up", _el(cfg), nw), c and c[0],
                                       _arg(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_expert_down(cfg, round_, w_down, ws, stream=None, counts_host=None,
                    n_rounds=1):
    c = _counts(counts_host)
    _check(load().moe_expert_down(ctypes.byref(cfg), int(round_), int(n_rounds),
                                  _arg(w_down, "w_down", _el(cfg),
                                       cfg.E * cfg.d_model * cfg.d_ff),
                                  c and c[0], _arg(ws, "ws"),
                                  _nbytes(ws), _stream(stream)))


def moe_pack_weights(cfg, w_gate, w_up, w_down, out_gate, out_up, out_down,
                     stream=None):
    """Row-major expert weights -> the tiled layout (MOE_WEIGHTS_TILED)."""
    nw, el = cfg.E * cfg.d_model * cfg.d_ff, _el(cfg)
    _check(load().moe_pack_weights(ctypes.byref(cfg), _arg(w_gate, "w_gate", el, nw),
                                   _arg(w_up, "w_up", el, nw),
                                   _arg(w_down, "w_down", el, nw),
                                   _arg(out_gate, "out_gate", el, nw),
                                   _arg(out_up, "out_up", el, nw),
                                   _arg(out_down, "out_down", el, nw), _stream(stream)))


def moe_combine(cfg, ws, y, stream=None):
    _check(load().moe_combine(ctypes.byref(cfg), _arg(ws, "ws"), _nbytes(ws),
                              _arg(y, "y", _el(cfg), cfg.T * cfg.d_model),
                              _stream(stream)))


def moe_forward(cfg, logits, x, w_gate, w_up, w_down, y, ws, stream=None):
    nw, el, nx = cfg.E * cfg.d_model * cfg.d_ff, _el(cfg), cfg.T * cfg.d_model
    _check(load().moe_forward(ctypes.byref(cfg),
                              _arg(logits, "logits", torch.float32, cfg.T * cfg.E),
                              _arg(x, "x", el, nx), _arg(w_gate, "w_gate", el, nw),
                              _arg(w_up, "w_up", el, nw), _arg(w_down, "w_down", el, nw),
                              _arg(y, "y", el, nx), _arg(ws, "ws"), _nbytes(ws),
                              _stream(stream)))


# bytes of the library's static workspace (MOE_STATIC_WORKSPACE_BYTES)
STATIC_WORKSPACE_BYTES = 64 << 20


def moe_forward_static(cfg, logits, x, w_gate, w_up, w_down, y, stream=None):
    """moe_forward on the library's static device workspace: the call
    allocates nothing (see moe_forward_static in the header)."""
    nw, el, nx = cfg.E * cfg.d_model * cfg.d_ff, _el(cfg), cfg.T * cfg.d_model
    _check(load().moe_forward_static(
        ctypes.byref(cfg), _arg(logits, "logits", torch.float32, cfg.T * cfg.E),
        _arg(x, "x", el, nx), _arg(w_gate, "w_gate", el, nw),
        _arg(w_up, "w_up", el, nw), _arg(w_down, "w_down", el, nw),
        _arg(y, "y", el, nx), _stream(stream)))


def backward_workspace_size(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_backward_workspace_size(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def backward_layout(cfg: MoeConfig) -> dict:
    L = MoeBackwardLayout()
    _check(load().moe_backward_layout(ctypes.byref(cfg), ctypes.byref(L)))
    return {n: getattr(L, n) for n in BWD_LAYOUT_FIELDS + ("total",)}


def moe_backward(cfg, x, w_gate, w_up, w_down, dy, dx, dlogits,
                 dw_gate, dw_up, dw_down, ws, bws, stream=None):
    """The layer's backward after moe_forward (ws: its workspace; the
    weights as given to moe_forward)."""
    nw, el, nx = cfg.E * cfg.d_model * cfg.d_ff, _el(cfg), cfg.T * cfg.d_model
    f32 = torch.float32
    _check(load().moe_backward(
        ctypes.byref(cfg), _arg(x, "x", el, nx), _arg(w_gate, "w_gate", el, nw),
        _arg(w_up, "w_up", el, nw), _arg(w_down, "w_down", el, nw),
        _arg(dy, "dy", el, nx),
        _arg(dx, "dx", el, nx), _arg(dlogits, "dlogits", f32, cfg.T * cfg.E),
        _arg(dw_gate, "dw_gate", f32, nw), _arg(dw_up, "dw_up", f32, nw),
        _arg(dw_down, "dw_down", f32, nw), _arg(ws, "ws"), _nbytes(ws),
        _arg(bws, "bws"), _nbytes(bws), _stream(stream)))


def _counts_rows(cfg: MoeConfig, counts):
    """Observed counts as a C-contiguous int32 [n_steps, E] array."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    if a.ndim == 1:
        a = a.reshape(1, -1)
    if a.ndim != 2 or a.shape[1] != cfg.E:
        raise ValueError(f"counts must be [n_steps, {cfg.E}]")
    return a


def capacity_curve(cfg: MoeConfig, counts, capacities):
    """(rounds [n_C, n_steps], workspace bytes [n_C]) for each capacity C:
    the memory-against-rounds curve of the observed steps' counts."""
    import numpy as np
    a = _counts_rows(cfg, counts)
    caps = np.ascontiguousarray(np.asarray(capacities, dtype=np.int64))
    rounds = np.zeros((caps.size, a.shape[0]), dtype=np.int32)
    ws = (ctypes.c_size_t * caps.size)()
    _check(load().moe_capacity_curve(
        ctypes.byref(cfg), a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        a.shape[0], caps.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        caps.size, rounds.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ws))
    return rounds, np.array(list(ws), dtype=np.int64)


def capacity_for_rounds(cfg: MoeConfig, counts, target_rounds=1,
                        quantile=1.0) -> int:
    """Smallest C with at most target_rounds rounds on a share `quantile` of
    the observed steps."""
    a = _counts_rows(cfg, counts)
    out = ctypes.c_int64(0)
    _check(load().moe_capacity_for_rounds(
        ctypes.byref(cfg), a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        a.shape[0], int(target_rounds), float(quantile), ctypes.byref(out)))
    return out.value


def workspace_views(cfg: MoeConfig, ws: torch.Tensor) -> dict:
    """torch views of the internal buffers of a uint8 workspace tensor.
    xr and h are returned as raw bytes of all sets of the round buffer (rows
    of d (f) elements in the tiled layout, see buffer_geometry); rounds is
    [9, M, E]: per (round, expert) rows, first index, rows of the group's
    lower experts, the same padded to 64, and the buffer row brow; then the
    pair tables indexed [b, v] (expert, rows, buffer row, first z row);
    round_pairs is [2, M]: rbeg and rend of every round."""
    L = workspace_layout(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    geo = buffer_geometry(cfg)
    rows, M = geo["rows"] * geo["S"], geo["M"]
    el = torch.bfloat16 if cfg.dtype == MOE_BF16 else torch.float32
    es = 2 if cfg.dtype == MOE_BF16 else 4

    def view(name, n, dt, size):
        return ws[L[name]:L[name] + n * size].view(dt)

    i32 = torch.int32
    return {
        "idx": view("idx", T * k, i32, 4).view(T, k),
        "weight": view("weight", T * k, torch.float32, 4).view(T, k),
        "counts": view("counts", E, i32, 4),
        "offsets": view("offsets", E + 1, i32, 4),
        "n_rounds": view("n_rounds", 1, i32, 4),
        "perm": view("perm", T * k, i32, 4),
        "pos": view("pos", T * k, i32, 4),
        "round_of": view("round_of", T * k, i32, 4),
        "row_of": view("row_of", T * k, i32, 4),
        "rounds": view("rounds", 9 * M * E, i32, 4).view(9, M, E),
        "round_pairs": ws[L["rounds"] + 36 * M * E:L["rounds"] + 36 * M * E + 8 * M]
        .view(i32).view(2, M),
        "xr": view("xr", rows * cfg.d_model * es, torch.uint8, 1),
        "h": view("h", rows * cfg.d_ff * es, torch.uint8, 1),
        "z": view("z", T * k * cfg.d_model, el, es).view(T * k, cfg.d_model),
    }
