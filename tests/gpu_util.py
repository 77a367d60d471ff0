"""Helpers for the GPU parity tests: upload seeded inputs, run the C ABI,
and compare with the oracle. Imported by GPU tests only."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import synth
from round_dropless_expert_amd.configs import Workload

# max |err| <= TOL * max |ref| over the compared elements
TOL = {"f32": 1e-4, "bf16": 2e-2}


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def el_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


class Case:
    """One workload's inputs on the host (float32, dtype-exact) and device."""

    def __init__(self, w: Workload, dev="cuda:0"):
        self.w = w
        self.dev = dev
        note(f"generate {w.name} T={w.T} d={w.d_model} f={w.d_ff} E={w.E} "
             f"k={w.k} C={w.C} skew={w.skew}")
        self.inp = synth.generate(w)
        dt = el_dtype(w)
        up = lambda a: torch.from_numpy(a).to(dev).to(dt).contiguous()
        self.logits = torch.from_numpy(self.inp.logits).to(dev)
        self.x = up(self.inp.x)
        self.wg = up(self.inp.Wg)
        self.wu = up(self.inp.Wu)
        self.wd = up(self.inp.Wd)
        self.idx, self.wt = oracle.route(self.inp.logits, w.k)

    def cfg(self, C=None, weight_layout="tiled", group=1, round_buffers=1):
        w = self.w
        return B.config(w.T, w.E, w.k, w.d_model, w.d_ff,
                        w.C if C is None else C, w.dtype, weight_layout, group,
                        round_buffers)

    def weights(self, layout="tiled"):
        """(w_gate, w_up, w_down) on the device in the given layout."""
        if layout == "row_major":
            return self.wg, self.wu, self.wd
        if not hasattr(self, "_packed"):
            out = [torch.empty_like(t) for t in (self.wg, self.wu, self.wd)]
            note(f"{self.w.name}: moe_pack_weights")
            B.moe_pack_weights(self.cfg(), self.wg, self.wu, self.wd, *out)
            torch.cuda.synchronize()
            self._packed = tuple(out)
        return self._packed

    def workspace(self, cfg, poison=True):
        n = B.workspace_size(cfg)
        ws = torch.empty(n, dtype=torch.uint8, device=self.dev)
        if poison:
            ws.fill_(0xFF)  # NaN in bf16 and fp32: unwritten slots show
        return ws

    def new_y(self):
        return torch.full((self.w.T, self.w.d_model), float("nan"),
                          dtype=el_dtype(self.w), device=self.dev)

    def oracle_y(self, tokens):
        return oracle.forward_tokens(tokens, self.idx, self.wt, self.inp.x,
                                     self.inp.Wg, self.inp.Wu, self.inp.Wd)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    scale = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (scale if scale > 0 else 1.0))


def assert_close(got, ref, dtype: str, what: str) -> float:
    e = rel_err(got, ref)
    assert e <= TOL[dtype], f"{what}: max|err|/max|ref| = {e:.3e} > {TOL[dtype]}"
    return e


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 \
        else t.detach().cpu().numpy()


def reference_placement(p: oracle.Plan, E: int, cfg):
    """The launch batches of a plan and where every (round, expert) matrix
    starts in the round buffer: with one capacity group per expert and one
    set of round buffers, consecutive rounds share a batch while their pairs
    (experts with rows) number at most E, and pair v of a batch starts at
    row v * P; otherwise each round is a batch and expert e's matrix starts
    at its group's block plus the padded rows of the group's lower experts.
    Returns (brow [R, E], pairs: list per batch of (r, e, m, brow, z row),
    rbeg [R], rend [R])."""
    geo = B.buffer_geometry(cfg)
    G, P, Q = geo["G"], geo["pad"], geo["Q"]
    pack = G == 1 and geo["S"] == 1
    brow = np.zeros((p.R, E), dtype=np.int64)
    batches, rbeg, rend = [], np.zeros(p.R, np.int64), np.zeros(p.R, np.int64)
    for r in range(p.R):
        m = p.rows_in_round(r)
        first = p.first_in_round(r)
        act = [e for e in range(E) if m[e] > 0]
        if not batches or not pack or len(batches[-1]) + len(act) > E:
            batches.append([])
        cur = batches[-1]
        b = len(batches) - 1
        rbeg[r] = b * E + len(cur)
        mp = (m + 63) // 64 * 64
        for e in range(E):
            g0 = e - e % G
            brow[r, e] = (e // G) * Q + mp[g0:e].sum()
        for e in act:
            if pack:
                brow[r, e] = len(cur) * P
            cur.append((r, e, int(m[e]), int(brow[r, e]),
                        int(p.offsets[e] + first[e])))
        rend[r] = b * E + len(cur)
    return brow, batches, rbeg, rend


def assert_plan_equal(views: dict, p: oracle.Plan, idx: np.ndarray, cfg=None):
    np.testing.assert_array_equal(views["idx"].cpu().numpy(), idx)
    np.testing.assert_array_equal(views["counts"].cpu().numpy(), p.counts)
    np.testing.assert_array_equal(views["offsets"].cpu().numpy(), p.offsets)
    np.testing.assert_array_equal(views["perm"].cpu().numpy(), p.perm)
    np.testing.assert_array_equal(views["pos"].cpu().numpy(), p.pos)
    np.testing.assert_array_equal(views["round_of"].cpu().numpy(), p.round_of)
    np.testing.assert_array_equal(views["row_of"].cpu().numpy(), p.row_of)
    assert int(views["n_rounds"].item()) == p.R
    # round tables: rows, first index, rows of the group's lower experts
    # (plain and padded to 64), from the oracle's allocation
    t = views["rounds"].cpu().numpy()[:, :p.R].astype(np.int64)
    E = p.counts.size
    for r in range(p.R):
        m = p.rows_in_round(r)
        np.testing.assert_array_equal(t[0, r], m)
        np.testing.assert_array_equal(t[1, r], p.first_in_round(r))
        mp = (m + 63) // 64 * 64
        for name, v, row in (("ubase", m, t[2, r]), ("pbase", mp, t[3, r])):
            ex = np.zeros(E, dtype=np.int64)
            for e in range(E):
                g0 = e - e % p.G
                ex[e] = v[g0:e].sum()
            np.testing.assert_array_equal(row, ex, err_msg=f"{name} round {r}")
    if cfg is None:
        return
    # launch batches: buffer rows of every active (round, expert), the pair
    # tables and each round's range of pairs
    brow, batches, rbeg, rend = reference_placement(p, E, cfg)
    full = views["rounds"].cpu().numpy().astype(np.int64)
    for r in range(p.R):
        act = p.rows_in_round(r) > 0
        np.testing.assert_array_equal(full[4, r][act], brow[r][act],
                                      err_msg=f"brow round {r}")
    rp = views["round_pairs"].cpu().numpy()[:, :p.R].astype(np.int64)
    np.testing.assert_array_equal(rp[0], rbeg, err_msg="rbeg")
    np.testing.assert_array_equal(rp[1], rend, err_msg="rend")
    flat = full[5:9].reshape(4, -1)
    for b, pairs in enumerate(batches):
        for v, (r, e, m, row, z) in enumerate(pairs):
            np.testing.assert_array_equal(flat[:, b * E + v], [e, m, row, z],
                                          err_msg=f"pair {v} of batch {b}")


def expert_rows(views: dict, cfg, r: int, e: int, m: int, cols: int, dtype,
                buf: str = "xr") -> torch.Tensor:
    """Rows 0..m-1 of expert e's matrix of round r in the xr (or h) round
    buffer: in set r % S it starts at row brow(r, e), padded to 64."""
    geo = B.buffer_geometry(cfg)
    es = torch.empty(0, dtype=dtype).element_size()
    rb = cols * es
    start = (r % geo["S"]) * geo["rows"] + int(views["rounds"][4, r, e].item())
    rows = (m + 63) // 64 * 64
    seg = views[buf][start * rb:(start + rows) * rb]
    return untile(seg, rows, cols, dtype)[:m]


def sample_tokens(T: int, p: oracle.Plan, k: int, n: int, seed: int = 1):
    """Tokens 0 and T-1, every token with an assignment in the last round
    (up to n), and a seeded random sample."""
    rng = np.random.default_rng(seed)
    last = np.unique(np.nonzero(p.round_of == p.R - 1)[0] // k)
    if last.size > n // 2:
        last = rng.choice(last, n // 2, replace=False)
    rand = rng.choice(T, min(T, n), replace=False)
    return np.unique(np.concatenate([[0, T - 1], last, rand])).astype(np.int64)


def tiled_index(rows: int, row_bytes: int) -> np.ndarray:
    """Byte offset, in the tiled layout (64-row x 64-byte blocks, chunk c of
    row r stored at c ^ ((r >> 2) & 3)), of every byte of a rows x row_bytes
    row-major matrix. rows must be a multiple of 64."""
    r = np.arange(rows, dtype=np.int64)[:, None]
    b = np.arange(row_bytes, dtype=np.int64)[None, :]
    blk = (r >> 6) * (row_bytes >> 6) + (b >> 6)
    rr = r & 63
    bb = b & 63
    return blk * 4096 + rr * 64 + (((bb >> 4) ^ ((rr >> 2) & 3)) << 4) + (bb & 15)


def untile(mat_bytes: torch.Tensor, rows: int, cols: int, dtype) -> torch.Tensor:
    """Row-major [rows, cols] tensor of `dtype` from one tiled matrix."""
    es = torch.empty(0, dtype=dtype).element_size()
    idx = torch.from_numpy(tiled_index(rows, cols * es)).to(mat_bytes.device)
    return mat_bytes[idx.reshape(-1)].view(rows, cols * es).view(dtype)


def tiled_rows(buf: torch.Tensor, rows: np.ndarray, cols: int, dtype) -> torch.Tensor:
    """Rows `rows` (row indices of one tiled matrix whose rows hold `cols`
    elements of `dtype`, stored in the byte tensor `buf`) as a row-major
    [len(rows), cols] tensor."""
    es = torch.empty(0, dtype=dtype).element_size()
    rb = cols * es
    r = np.asarray(rows, dtype=np.int64)[:, None]
    b = np.arange(rb, dtype=np.int64)[None, :]
    blk = (r >> 6) * (rb >> 6) + (b >> 6)
    rr = r & 63
    bb = b & 63
    off = blk * 4096 + rr * 64 + (((bb >> 4) ^ ((rr >> 2) & 3)) << 4) + (bb & 15)
    idx = torch.from_numpy(off.reshape(-1)).to(buf.device)
    return buf[idx].view(len(rows), rb).view(dtype)
