"""ctypes wrapper of the CPU oracle (fp64, plain C).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and
the benchmark's CPU-baseline leg, never by the HIP library or its binding.
It shares no code with the HIP path; both are fed by the seeded input
generator, which holds none of the layer's arithmetic.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

from .build import LIB as _LIB, build as _build

_lib = None

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class OracleError(RuntimeError):
    pass


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            _build()
        L = ctypes.CDLL(_LIB)
        L.oracle_route.argtypes = [_i64, _i32, _i32, _f32p, _i32p, _f64p]
        L.oracle_plan.argtypes = [_i64, _i32, _i32, _i64, _i32p, _i32p, _i32p,
                                  _i32p, _i32p, _i32p, _i32p, _i32p]
        L.oracle_assignment_outputs.argtypes = [
            _i64, _i32, _i32, _i32, _i32, _i64, _i64p, _i32p, _f32p, _f32p,
            _f32p, _f32p, ctypes.c_void_p, _f64p]
        L.oracle_forward_tokens.argtypes = [
            _i64, _i32, _i32, _i32, _i32, _i64, _i64p, _i32p, _f64p, _f32p,
            _f32p, _f32p, _f32p, _f64p]
        L.oracle_round_executor.argtypes = [
            _i64, _i32, _i32, _i32, _i32, _i64, _i32p, _f64p, _i32p, _i32p,
            _i32p, _i32p, _i32p, _i32, _f32p, _f32p, _f32p, _f32p, _f64p,
            _f64p]
        L.oracle_plan_groups.argtypes = [
            _i64, _i32, _i32, _i64, _i32, _i32p, _i32p, _i32p, _i32p, _i32p,
            _i32p, _i32p, _i32p, _i32p, _i64]
        L.oracle_round_executor_groups.argtypes = [
            _i64, _i32, _i32, _i32, _i32, _i64, _i32, _i32p, _f64p, _i32p,
            _i32p, _i32p, _i32p, _i32p, _i32, _i32p, _f32p, _f32p, _f32p,
            _f32p, _f64p, _f64p]
        L.oracle_backward_tokens.argtypes = [
            _i64, _i32, _i32, _i32, _i32, _i64, _i64p, _i32p, _f64p, _f32p,
            _f32p, _f32p, _f32p, _f32p, _f64p, _f64p]
        L.oracle_weight_grads.argtypes = [
            _i64, _i32, _i32, _i32, _i32, _i32, _i32p, _f64p, _f32p, _f32p,
            _f32p, _f32p, _f32p, _f64p, _f64p, _f64p]
        for name in ("oracle_route", "oracle_plan", "oracle_assignment_outputs",
                     "oracle_backward_tokens", "oracle_weight_grads",
                     "oracle_forward_tokens", "oracle_round_executor",
                     "oracle_plan_groups", "oracle_round_executor_groups",
                     "oracle_max_threads"):
            getattr(L, name).restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def max_threads() -> int:
    return lib().oracle_max_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def route(logits: np.ndarray, k: int):
    """Top-k routing: idx int32 [T, k] and weights fp64 [T, k]."""
    logits = _f32(logits)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    _check(lib().oracle_route(T, E, k, logits, idx, w), "oracle_route")
    return idx, w


@dataclasses.dataclass
class Plan:
    counts: np.ndarray    # int32 [E]
    offsets: np.ndarray   # int32 [E+1]
    perm: np.ndarray      # int32 [T*k]
    pos: np.ndarray       # int32 [T*k]
    round_of: np.ndarray  # int32 [T*k]
    row_of: np.ndarray    # int32 [T*k]
    R: int
    C_eff: int
    G: int = 1                 # experts per capacity group
    alloc: np.ndarray = None   # int32 [R, E] rows per round (groups only)

    def rows_in_round(self, r: int) -> np.ndarray:
        """m_{r,e} for every expert (int64 [E])."""
        if self.alloc is not None:
            return self.alloc[r].astype(np.int64)
        m = self.counts.astype(np.int64) - r * self.C_eff
        return np.clip(m, 0, self.C_eff)

    def first_in_round(self, r: int) -> np.ndarray:
        """Index, in each expert's stable list, of its first round-r entry."""
        if self.alloc is not None:
            return self.alloc[:r].astype(np.int64).sum(axis=0)
        return np.minimum(self.counts.astype(np.int64), r * self.C_eff)


def plan(idx: np.ndarray, E: int, C: int) -> Plan:
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    TK = T * k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(TK, dtype=np.int32)
    pos = np.empty(TK, dtype=np.int32)
    round_of = np.empty(TK, dtype=np.int32)
    row_of = np.empty(TK, dtype=np.int32)
    R = np.zeros(1, dtype=np.int32)
    _check(lib().oracle_plan(T, E, k, C, idx.reshape(-1), counts, offsets,
                             perm, pos, round_of, row_of, R), "oracle_plan")
    return Plan(counts, offsets, perm, pos, round_of, row_of, int(R[0]),
                min(int(C), int(T)))


def plan_groups(idx: np.ndarray, E: int, C: int, G: int) -> Plan:
    """Plan with the capacity of each group of G experts shared among them
    (oracle_plan_groups); G = 1 is the strict per-expert capacity."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    TK = T * k
    Ce = min(int(C), int(T))
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(TK, dtype=np.int32)
    pos = np.empty(TK, dtype=np.int32)
    round_of = np.empty(TK, dtype=np.int32)
    row_of = np.empty(TK, dtype=np.int32)
    R = np.zeros(1, dtype=np.int32)
    rows = -(-T // Ce)  # at most ceil(T / C') rounds
    alloc = np.zeros(rows * E, dtype=np.int32)
    _check(lib().oracle_plan_groups(T, E, k, C, G, idx.reshape(-1), counts,
                                    offsets, perm, pos, round_of, row_of, R,
                                    alloc, rows), "oracle_plan_groups")
    R = int(R[0])
    return Plan(counts, offsets, perm, pos, round_of, row_of, R, Ce, int(G),
                alloc.reshape(rows, E)[:R].copy())


def round_executor_groups(idx, w, p: Plan, C: int, x, Wg, Wu, Wd):
    """round_executor for a plan_groups plan."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, k = idx.shape
    E, f, d = Wg.shape
    Z = np.empty((T * k, d), dtype=np.float64)
    y = np.empty((T, d), dtype=np.float64)
    alloc = np.ascontiguousarray(p.alloc, dtype=np.int32).reshape(-1)
    if alloc.size == 0:
        alloc = np.zeros(1, dtype=np.int32)
    _check(lib().oracle_round_executor_groups(
        T, E, k, d, f, C, p.G, idx.reshape(-1), w.reshape(-1), p.counts,
        p.offsets, p.perm, p.round_of, p.row_of, p.R, alloc, _f32(x),
        _f32(Wg), _f32(Wu), _f32(Wd), Z, y), "oracle_round_executor_groups")
    return Z, y


def assignment_outputs(a_list, idx, x, Wg, Wu, Wd, want_h=False):
    """Expert FFN outputs for the listed assignments: (h [n,f] or None,
    o [n,d]) in fp64."""
    a_list = np.ascontiguousarray(a_list, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    E, f, d = Wg.shape
    n = a_list.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    h = np.empty((n, f), dtype=np.float64) if want_h else None
    _check(lib().oracle_assignment_outputs(
        T, E, k, d, f, n, a_list, idx.reshape(-1), _f32(x), _f32(Wg),
        _f32(Wu), _f32(Wd), h.ctypes.data if h is not None else None, o),
        "oracle_assignment_outputs")
    return h, o


def forward_tokens(tokens, idx, w, x, Wg, Wu, Wd) -> np.ndarray:
    """Layer output rows y [n, d] (fp64) for the listed tokens, by the plain
    per-token loop over each token's top-k experts."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, k = idx.shape
    E, f, d = Wg.shape
    n = tokens.shape[0]
    y = np.empty((n, d), dtype=np.float64)
    _check(lib().oracle_forward_tokens(
        T, E, k, d, f, n, tokens, idx.reshape(-1), w.reshape(-1), _f32(x),
        _f32(Wg), _f32(Wu), _f32(Wd), y), "oracle_forward_tokens")
    return y


def round_executor(idx, w, p: Plan, C: int, x, Wg, Wu, Wd):
    """Run the plan round by round through a fixed E x C buffer; returns
    (Z [T*k, d], y [T, d]) in fp64."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    T, k = idx.shape
    E, f, d = Wg.shape
    Z = np.empty((T * k, d), dtype=np.float64)
    y = np.empty((T, d), dtype=np.float64)
    _check(lib().oracle_round_executor(
        T, E, k, d, f, C, idx.reshape(-1), w.reshape(-1), p.counts, p.offsets,
        p.perm, p.round_of, p.row_of, p.R, _f32(x), _f32(Wg), _f32(Wu),
        _f32(Wd), Z, y), "oracle_round_executor")
    return Z, y


def backward_tokens(tokens, idx, w, x, Wg, Wu, Wd, dy):
    """Gradients of L = sum_t <y_t, dy_t> for a list of tokens: dx [n, d]
    and dlogits [n, E] (fp64)."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    x, Wg, Wu, Wd, dy = (_f32(a) for a in (x, Wg, Wu, Wd, dy))
    T, d = x.shape
    E, f, _ = Wg.shape
    k = idx.shape[1]
    n = tokens.size
    dx = np.empty((n, d), dtype=np.float64)
    dl = np.empty((n, E), dtype=np.float64)
    _check(lib().oracle_backward_tokens(
        T, E, k, d, f, n, tokens, np.ascontiguousarray(idx, dtype=np.int32),
        np.ascontiguousarray(w, dtype=np.float64), x, Wg, Wu, Wd, dy, dx, dl),
        "oracle_backward_tokens")
    return dx, dl


def weight_grads(e, idx, w, x, Wg, Wu, Wd, dy):
    """Weight gradients of expert e: dWg, dWu [f, d] and dWd [d, f] (fp64)."""
    x, Wg, Wu, Wd, dy = (_f32(a) for a in (x, Wg, Wu, Wd, dy))
    T, d = x.shape
    E, f, _ = Wg.shape
    k = idx.shape[1]
    dWg = np.empty((f, d), dtype=np.float64)
    dWu = np.empty((f, d), dtype=np.float64)
    dWd = np.empty((d, f), dtype=np.float64)
    _check(lib().oracle_weight_grads(
        T, E, k, d, f, int(e), np.ascontiguousarray(idx, dtype=np.int32),
        np.ascontiguousarray(w, dtype=np.float64), x, Wg, Wu, Wd, dy, dWg, dWu,
        dWd), "oracle_weight_grads")
    return dWg, dWu, dWd
