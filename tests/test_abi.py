"""The C ABI on the CPU: the library loads, exports every function the header
declares, computes the workspace layout as a pure function of the config, and
rejects bad arguments with exact status codes before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_rounds.h")


@pytest.fixture(scope="module")
def B():
    from round_dropless_expert_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from round_dropless_expert_amd.csrc import build
        build.build()
    binding.load()
    return binding


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n;]*?\b(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_plan", "moe_dispatch", "moe_expert_ffn", "moe_combine",
              "moe_forward", "moe_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    L = B.load()
    names = declared_functions()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)$", out, re.M))
    assert set(names) <= exported
    assert set(B.EXPORTS) == set(names)


def ceil_div(a, b):
    return -(-a // b)


def expected_total(T, E, k, d, f, C, es, G=1, S=1):
    al = lambda v: (v + 255) // 256 * 256
    ce = min(C, T)
    pad = ceil_div(ce, 64) * 64  # round-buffer rows per expert, tiled
    Q = pad if G == 1 else G * (pad + 64)  # rows per capacity group
    rows = E // G * Q
    M = ceil_div(T, ce)  # rounds at most
    TK = T * k
    nb = ceil_div(T, 8) + ceil_div(T, 256)  # plan histogram rows, chunk sums
    # counts and R share one block: [E counts][R]
    parts = [TK * 4, TK * 4, (E + 1) * 4, (E + 1) * 4, TK * 4, TK * 4, TK * 4,
             TK * 4, (9 * M * E + 2 * M) * 4, nb * E * 4, S * rows * d * es,
             S * rows * f * es,
             TK * d * es]
    return sum(al(p) for p in parts)


def test_workspace_is_a_function_of_the_config_only(B):
    from round_dropless_expert_amd import configs
    sizes = {}
    for name, w in configs.WORKLOADS.items():
        cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype)
        es = 2 if w.dtype == "bf16" else 4
        n = B.workspace_size(cfg)
        assert n == expected_total(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, es)
        lay = B.workspace_layout(cfg)
        assert lay["n_rounds"] == lay["counts"] + 4 * w.E
        # the documented order, the round buffer xr last
        order = ("idx", "weight", "counts", "offsets", "perm", "pos", "round_of",
                 "row_of", "rounds", "scratch", "h", "z", "xr")
        offs = [lay[f] for f in order]
        assert all(o % 256 == 0 for o in offs)
        assert offs == sorted(offs) and lay["total"] == n
        # the forward gathers its rows from x (at most 2^30 bytes here), so
        # it and the backward need only the workspace before xr
        assert w.T * w.d_model * es <= 1 << 30
        assert B.forward_workspace_size(cfg) == lay["xr"]
        sizes[name] = n
    # skewed routing needs exactly the balanced workload's memory
    assert sizes["skewed_bf16"] == sizes["balanced_bf16"]
    assert 336_000_000 < sizes["balanced_bf16"] < 337_000_000
    # group 0 means 1
    w = configs.BALANCED_BF16
    assert B.workspace_size(B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, "bf16",
                                     group=0)) == sizes["balanced_bf16"]
    # capacity costs memory; above T it acts as T
    w = configs.HOT_EXPERT_BF16
    prev = 0
    for C in w.sweep_C:
        n = B.workspace_size(B.config(w.T, w.E, w.k, w.d_model, w.d_ff, C, "bf16"))
        assert n > prev
        prev = n
    big = B.workspace_size(B.config(w.T, w.E, w.k, w.d_model, w.d_ff, 10 * w.T, "bf16"))
    assert big == prev
    # capacity groups: G*(P+64) rows per group of G experts
    for G in (2, 4, 64):
        n = B.workspace_size(B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C,
                                      "bf16", group=G))
        assert n == expected_total(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, 2, G)
    # two sets of round buffers: one more xr and h; 0 means 1
    for G in (1, 4):
        one = B.workspace_size(B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C,
                                        "bf16", group=G, round_buffers=0))
        two = B.workspace_size(B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C,
                                        "bf16", group=G, round_buffers=2))
        assert two == expected_total(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, 2,
                                     G, 2)
        geo = B.buffer_geometry(B.config(w.T, w.E, w.k, w.d_model, w.d_ff,
                                         w.C, "bf16", group=G))
        assert two - one == geo["rows"] * (w.d_model + w.d_ff) * 2


BAD_CONFIGS = [
    (dict(T=0), 1), (dict(E=0), 1), (dict(k=0), 1), (dict(k=9), 1),
    (dict(C=0), 1), (dict(d_model=0), 1), (dict(dtype=7), 1),
    (dict(weight_layout=2), 1), (dict(group=3), 1), (dict(group=-1), 1),
    (dict(round_buffers=3), 1), (dict(round_buffers=-1), 1),
    (dict(E=65, k=2), 2), (dict(d_model=96), 2), (dict(d_ff=100), 2),
    (dict(T=1 << 29, k=4), 2),
]


@pytest.mark.parametrize("change,status", BAD_CONFIGS)
def test_config_validation(B, change, status):
    base = dict(T=512, E=8, k=2, d_model=64, d_ff=128, C=64, dtype=0,
                weight_layout=0, group=1, round_buffers=1)
    base.update(change)
    cfg = B.config(**base)
    assert B.check_config(cfg) == status
    L = B.load()
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)) == status
    assert B.load().moe_last_error().decode()


def test_null_config(B):
    L = B.load()
    n = ctypes.c_size_t(0)
    assert L.moe_workspace_size(None, ctypes.byref(n)) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_forward(None, 16, 16, 16, 16, 16, 16, 16, 1 << 40, None) == \
        B.MOE_ERR_INVALID_ARGUMENT


def test_pointer_and_workspace_checks_before_any_hip_call(B):
    """These calls fail validation, so they never reach the HIP runtime (this
    machine has no GPU: a HIP call would report an error of its own)."""
    L = B.load()
    cfg = B.config(512, 8, 2, 64, 128, 64, "f32")
    need = B.workspace_size(cfg)
    p = 1 << 20  # aligned fake device address, never dereferenced
    c = ctypes.byref(cfg)
    assert L.moe_forward(c, p, p, p, p, p, p, p, B.forward_workspace_size(cfg) - 1,
                         None) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_forward(c, p, p, p, p, p, p, None, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_forward(c, p + 4, p, p, p, p, p, p, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_forward(c, p, p, p, p, None, p, p, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_plan(c, None, p, need, None, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_plan(c, p, p + 8, need, None, None) == B.MOE_ERR_INVALID_ARGUMENT
    # round range: ceil(T / C') rounds at most
    assert L.moe_dispatch(c, -1, 1, p, p, need, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_dispatch(c, 8, 1, p, p, need, None) == B.MOE_ERR_INVALID_ARGUMENT
    # a round range: n_rounds >= 1 and round + n_rounds <= ceil(T / C')
    assert L.moe_dispatch(c, 0, 0, p, p, need, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_dispatch(c, 5, 4, p, p, need, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_expert_ffn(c, 8, 1, p, p, p, None, p, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_expert_ffn(c, 7, 2, p, p, p, None, p, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_expert_gate_up(c, 0, 1, p, None, None, p, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_expert_down(c, -1, 1, p, None, p, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_dispatch_gate_up(c, 0, 1, None, p, p, None, p, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_dispatch_gate_up(c, 8, 1, p, p, p, None, p, need, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_dispatch_gate_up(c, 0, 1, p, p, p, None, p, need - 1, None) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    # x of more than 2^30 bytes: the gathering launch is refused (the forward
    # dispatches such an x into the round buffer instead, so it needs all of
    # the workspace)
    huge = B.config(1 << 19, 8, 2, 2048, 128, 1 << 16, "bf16")
    assert huge.T * huge.d_model * 2 > 1 << 30
    assert L.moe_dispatch_gate_up(ctypes.byref(huge), 0, 1, p, p, p, None, p,
                                  B.workspace_size(huge), None) == B.MOE_ERR_UNSUPPORTED
    assert b"2^30" in L.moe_last_error()
    assert B.forward_workspace_size(huge) == B.workspace_size(huge)
    # the forward and the backward accept the workspace before xr; the stage
    # calls need all of it
    fwd = B.forward_workspace_size(cfg)
    assert fwd == B.workspace_layout(cfg)["xr"] < need
    assert L.moe_forward(c, p, p, p, p, p, p, p, fwd - 1, None) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_forward(c, p, p, p, p, None, p, p, fwd, None) == \
        B.MOE_ERR_INVALID_ARGUMENT  # past the size check: a NULL pointer
    assert L.moe_dispatch(c, 0, 1, p, p, fwd, None) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_expert_ffn(c, 0, 1, p, p, p, None, p, fwd, None) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_forward_workspace_size(c, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_combine(c, p, need, None, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_pack_weights(c, p, p, None, p, p, p, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"


def test_static_forward_checks_before_any_hip_call(B):
    """moe_forward_static rejects a config whose workspace exceeds the
    static one, and bad pointers, before any HIP call."""
    L = B.load()
    m = re.search(r"#define MOE_STATIC_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == B.STATIC_WORKSPACE_BYTES
    p = 1 << 20
    big = B.config(8192, 32, 4, 2048, 1024, 1024, "bf16")
    assert B.forward_workspace_size(big) > B.STATIC_WORKSPACE_BYTES
    assert L.moe_forward_static(ctypes.byref(big), p, p, p, p, p, p, None) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert b"static workspace" in L.moe_last_error()
    small = B.config(512, 8, 2, 64, 128, 64, "f32")
    c = ctypes.byref(small)
    assert L.moe_forward_static(c, p, p, p, p, p, None, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_forward_static(c, p, p + 4, p, p, p, p, None) == \
        B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_forward_static(None, p, p, p, p, p, p, None) == \
        B.MOE_ERR_INVALID_ARGUMENT


def expected_backward_total(T, E, k, d, f, C, G=1):
    al = lambda v: (v + 255) // 256 * 256
    ce = min(C, T)
    pad = ceil_div(ce, 64) * 64
    Q = pad if G == 1 else G * (pad + 64)
    rows = E // G * Q
    TK = T * k
    # xr, dyr, hw and dgu in two sets (a pair of rounds), gu in one
    parts = [2 * rows * d * 2, 2 * rows * d * 2, rows * 2 * f * 2, 2 * rows * f * 2,
             2 * rows * 2 * f * 2, TK * d * 2, TK * 4]
    return sum(al(p) for p in parts)


def test_backward_workspace_is_a_function_of_the_config_only(B):
    from round_dropless_expert_amd import configs
    for name, w in configs.WORKLOADS.items():
        for G in (1, 2):
            cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, group=G)
            if w.dtype != "bf16":
                with pytest.raises(B.MoeError):
                    B.backward_workspace_size(cfg)
                continue
            n = B.backward_workspace_size(cfg)
            assert n == expected_backward_total(w.T, w.E, w.k, w.d_model, w.d_ff,
                                                w.C, G)
            lay = B.backward_layout(cfg)
            offs = [lay[f] for f in B.BWD_LAYOUT_FIELDS]
            assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
            assert lay["total"] == n


def test_backward_argument_checks_before_any_hip_call(B):
    L = B.load()
    cfg = B.config(512, 8, 2, 64, 128, 64, "bf16")
    need = B.workspace_size(cfg)
    bneed = B.backward_workspace_size(cfg)
    p = 1 << 20
    c = ctypes.byref(cfg)
    ptrs = [p] * 10  # x, w_gate, w_up, w_down, dy, dx, dlogits, dw_gate/up/down
    assert L.moe_backward(c, *ptrs, p, need, p, bneed - 1, None) == \
        B.MOE_ERR_WORKSPACE_TOO_SMALL
    # the forward's workspace up to xr is enough
    assert L.moe_backward(c, *ptrs, p, B.forward_workspace_size(cfg) - 1, p, bneed,
                          None) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    for i in range(10):
        bad = list(ptrs)
        bad[i] = None
        assert L.moe_backward(c, *bad, p, need, p, bneed, None) == \
            B.MOE_ERR_INVALID_ARGUMENT, i
    bad = list(ptrs)
    bad[5] = p + 2  # dx misaligned
    assert L.moe_backward(c, *bad, p, need, p, bneed, None) == B.MOE_ERR_INVALID_ARGUMENT
    f32 = B.config(512, 8, 2, 64, 128, 64, "f32")
    assert L.moe_backward(ctypes.byref(f32), *ptrs, p, need, p, bneed, None) == \
        B.MOE_ERR_UNSUPPORTED
    # k up to E is a valid forward config; the backward takes k <= 8
    k9 = B.config(512, 16, 9, 64, 128, 64, "bf16")
    assert B.check_config(k9) == B.MOE_OK
    assert L.moe_backward(ctypes.byref(k9), *ptrs, p, need, p, bneed, None) == \
        B.MOE_ERR_UNSUPPORTED
    assert "k <= 8" in L.moe_last_error().decode()
    with pytest.raises(B.MoeError):
        B.backward_workspace_size(k9)


def test_binding_rejects_host_tensors_before_the_library(B):
    """A host tensor would reach a kernel as a host address: the binding
    refuses it (no HIP call is made, so this runs without a GPU)."""
    import torch
    T, E, k, d, f = 64, 4, 2, 64, 128
    cfg = B.config(T, E, k, d, f, 64, "bf16")
    ws = torch.empty(B.workspace_size(cfg), dtype=torch.uint8)
    logits = torch.zeros(T, E)
    x = torch.zeros(T, d, dtype=torch.bfloat16)
    w = torch.zeros(E, f, d, dtype=torch.bfloat16)
    wd = torch.zeros(E, d, f, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    with pytest.raises(ValueError, match="cuda"):
        B.moe_forward(cfg, logits, x, w, w, wd, y, ws)
    with pytest.raises(ValueError, match="cuda"):
        B.moe_plan(cfg, logits, ws)
    with pytest.raises(ValueError, match="cuda"):
        B.moe_pack_weights(cfg, w, w, wd, w, w, wd)
    with pytest.raises(TypeError):
        B.moe_forward(cfg, logits.numpy(), x, w, w, wd, y, ws)


def test_calibration_library_loads_and_checks_arguments():
    """The benchmark's matrix-core calibration kernel lives in a library of
    its own (not the layer's ABI); it loads without a GPU and refuses bad
    arguments before any HIP call."""
    from round_dropless_expert_amd.csrc import build as hip_build
    L = ctypes.CDLL(hip_build.CALIB_LIB)
    f = L.moe_calibrate_mfma_bf16
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    p = 1 << 20
    hip_error_invalid_value = 1
    assert f(None, p, 8, 1, None) == hip_error_invalid_value
    assert f(p, None, 8, 1, None) == hip_error_invalid_value
    assert f(p, p, 0, 1, None) == hip_error_invalid_value
    assert f(p, p, 8, 0, None) == hip_error_invalid_value
