"""moe_forward_static, the entry point that allocates nothing, against
moe_forward through the C ABI: bit-identical y on two calls in a row (the
second with a smaller input, so the static workspace still holds the first
call's larger contents), no device memory taken by either call, and a config
too large for the static workspace rejected before anything runs."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import Case, assert_close, note, to_np
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import configs

pytestmark = pytest.mark.gpu

# a bf16 slice of the balanced shapes (2 rounds at C = 64), then a bf16 case
# with capacity groups and two round-buffer sets, then the tiny fp32
# workload (3 rounds): each call's workspace smaller than the one before
CALLS = [
    (dataclasses.replace(configs.BALANCED_BF16, name="balanced_slice", T=1000, C=64), 1, 1),
    (configs.Workload("groups_bf16", T=300, d_model=192, d_ff=320, E=6, k=3, C=40,
                      dtype="bf16", skew=("zipf", 1.0)), 2, 2),
    (configs.TINY_F32, 1, 1),
]


def _bits(y):
    return y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)


def test_static_forward_matches_moe_forward_twice():
    ref_bytes = None
    for i, (w, G, S) in enumerate(CALLS):
        case = Case(w)
        cfg = case.cfg(group=G, round_buffers=S)
        assert B.forward_workspace_size(cfg) <= B.STATIC_WORKSPACE_BYTES
        wg, wu, wd = case.weights()
        ws = case.workspace(cfg)
        y_ref = case.new_y()
        note(f"call {i}: {w.name} G={G} S={S}: moe_forward")
        B.moe_forward(cfg, case.logits, case.x, wg, wu, wd, y_ref, ws)
        torch.cuda.synchronize()
        del ws
        torch.cuda.empty_cache()
        y = case.new_y()
        torch.cuda.synchronize()
        alloc0 = torch.cuda.memory_allocated()
        free0, _ = torch.cuda.mem_get_info()
        note(f"call {i}: {w.name} G={G} S={S}: moe_forward_static")
        B.moe_forward_static(cfg, case.logits, case.x, wg, wu, wd, y)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        assert torch.cuda.memory_allocated() == alloc0
        if i > 0:  # the first call on the device may load the library's code
            assert free1 == free0, f"device memory changed by {free0 - free1} bytes"
        assert torch.equal(_bits(y), _bits(y_ref)), f"{w.name}: differs from moe_forward"
        # and against the oracle on every token (the bar moe_forward meets)
        assert_close(to_np(y), case.oracle_y(np.arange(w.T)), w.dtype, f"y of {w.name}")
        if ref_bytes is not None:
            assert B.forward_workspace_size(cfg) < ref_bytes, \
                "each call smaller than the last"
        ref_bytes = B.forward_workspace_size(cfg)


def test_static_forward_rejects_a_config_beyond_the_static_workspace():
    w = configs.BALANCED_BF16
    cfg = B.config(w.T, w.E, w.k, w.d_model, w.d_ff, w.C, w.dtype, "tiled")
    assert B.forward_workspace_size(cfg) > B.STATIC_WORKSPACE_BYTES
    dev = "cuda:0"
    logits = torch.zeros(w.T, w.E, device=dev)
    x = torch.zeros(w.T, w.d_model, dtype=torch.bfloat16, device=dev)
    wt = torch.zeros(w.E, w.d_ff, w.d_model, dtype=torch.bfloat16, device=dev)
    y = torch.full((w.T, w.d_model), 7.0, dtype=torch.bfloat16, device=dev)
    note("moe_forward_static: config beyond the static workspace")
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_static(cfg, logits, x, wt, wt, wt, y)
    assert ei.value.status == B.MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "y written by a rejected call"
