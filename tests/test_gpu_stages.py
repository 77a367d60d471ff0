"""Stage-by-stage parity of the HIP path with the oracle, through the C ABI:
route and plan bit-exact, dispatch bit-exact, the round's SwiGLU activations
and expert outputs within tolerance, and the combined output within
tolerance. Sizes span several tiles, ragged tails and partial feature
tiles, and finish in seconds on the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (Case, assert_close, assert_plan_equal, note, to_np)
from round_dropless_expert_amd import binding as B
from round_dropless_expert_amd import configs

pytestmark = pytest.mark.gpu

W = configs.Workload
STAGE_CASES = [
    configs.TINY_F32,
    # ragged slice of the balanced shapes: 125-row experts, 2 rounds at C=64
    dataclasses.replace(configs.BALANCED_BF16, name="balanced_slice", T=1000,
                        C=64),
    # several token tiles per expert, Zipf skew, 2+ rounds
    W("multi_tile_bf16", T=3000, d_model=512, d_ff=768, E=6, k=2, C=700,
      dtype="bf16", skew=("zipf", 1.0)),
    # feature sizes that leave partial feature tiles (d=192, f=320)
    W("partial_tiles_bf16", T=777, d_model=192, d_ff=320, E=5, k=3, C=100,
      dtype="bf16", skew=("zipf", 0.5)),
    W("partial_tiles_f32", T=300, d_model=192, d_ff=320, E=5, k=3, C=41,
      dtype="f32"),
    # single expert, k = 1: every token in one expert, C = 1 slot... small
    W("single_expert_bf16", T=200, d_model=128, d_ff=128, E=1, k=1, C=64,
      dtype="bf16"),
    # k = E (dense soft MoE)
    W("k_equals_E_bf16", T=150, d_model=256, d_ff=256, E=4, k=4, C=50,
      dtype="bf16"),
]


@pytest.mark.parametrize("w", STAGE_CASES, ids=lambda w: w.name)
def test_stages_match_oracle(w):
    torch.cuda.synchronize()
    case = Case(w)
    cfg = case.cfg()
    ws = case.workspace(cfg)
    note(f"{w.name}: moe_plan")
    R = B.moe_plan(cfg, case.logits, ws)
    views = B.workspace_views(cfg, ws)
    p = oracle.plan(case.idx, w.E, w.C)
    assert R == p.R
    assert_plan_equal(views, p, case.idx)
    wt = views["weight"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(wt - case.wt) <= 1e-6 * case.wt), "routing weights"

    ce = p.C_eff
    xr_bits = views["xr"].view(torch.int16 if w.dtype == "bf16" else torch.int32)
    x_bits = case.x.view(torch.int16 if w.dtype == "bf16" else torch.int32)
    for r in range(R):
        note(f"{w.name}: moe_dispatch round {r}")
        B.moe_dispatch(cfg, r, case.x, ws)
        torch.cuda.synchronize()
        m = p.rows_in_round(r)
        rows, assigns = [], []
        for e in range(w.E):
            for c in range(int(m[e])):
                rows.append(e * ce + c)
                assigns.append(int(p.perm[p.offsets[e] + r * ce + c]))
        rows_t = torch.tensor(rows, device=case.dev, dtype=torch.long)
        a_t = torch.tensor(assigns, device=case.dev, dtype=torch.long)
        assert torch.equal(xr_bits[rows_t], x_bits[a_t // w.k]), f"xr round {r}"

        note(f"{w.name}: moe_expert_ffn round {r}")
        B.moe_expert_ffn(cfg, r, case.wg, case.wu, case.wd, ws)
        torch.cuda.synchronize()
        h_ref, o_ref = oracle.assignment_outputs(
            np.array(assigns), case.idx, case.inp.x, case.inp.Wg, case.inp.Wu,
            case.inp.Wd, want_h=True)
        assert_close(to_np(views["h"][rows_t]), h_ref, w.dtype, f"h round {r}")
        assert_close(to_np(views["z"][a_t]), o_ref, w.dtype, f"z round {r}")

    note(f"{w.name}: moe_combine")
    y = case.new_y()
    B.moe_combine(cfg, ws, y)
    torch.cuda.synchronize()
    y_ref = case.oracle_y(np.arange(w.T))
    assert_close(to_np(y), y_ref, w.dtype, "y")
