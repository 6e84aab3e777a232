"""GPU parity of one GPU's share of expert parallelism (moe_permute_local).

A 16-expert layer is split into four shares of four experts.  For each share
the index (counts, offsets, dst_row, src_tok) and the dispatched rows must be
bit-exact against the oracle's share (local_expert_ids + build_index); each
share runs its own GroupedGEMM on its slice of the weights and a partial
combine in fp32; the four partials added together (the reduce-scatter's sum,
done here on the host as a stand-in for the collective) must match the
oracle's layer output within the bf16 layer bar (2e-2 * rms; the expert
outputs and the partial sums are fp32).  Routing is fed the oracle's fp32
logits.
"""
import numpy as np
import pytest
import torch

import moe_synth
from moe_synth import to_f32
from oracle import moe_ref as ref

from test_gpu_parity import DEV, check_close, dev_tensor, host, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_layer_24_amd import ops
    from mixture_experts_layer_24_amd._lib import MOE_BF16, MOE_F32


@pytest.mark.parametrize("T,h,hf,E,k,n", [(600, 256, 256, 16, 2, 4), (333, 128, 256, 8, 3, 2),
                                          (257, 128, 128, 6, 2, 3)])
def test_expert_parallel_shares(T, h, hf, E, k, n):
    wl = moe_synth.WORKLOADS["mixtral"].scaled(name="ep", T=T, h=h, h_ffn=hf, E=E, k=k)
    inp = moe_synth.gen_all(wl, seed=21)
    f = lambda key: to_f32(inp[key])
    fw = ref.layer_forward(f("x"), f("w_gate"), inp["bias"], f("w1"), f("w3"), f("w2"), k)
    xd = dev_tensor(inp["x"])
    idx = torch.from_numpy(fw["idx"].astype(np.int32)).to(DEV)
    w = torch.from_numpy(fw["w"].astype(np.float32)).to(DEV)
    total = np.zeros((T, h))
    for r in range(n):
        e_lo, e_cnt = r * E // n, (r + 1) * E // n - r * E // n
        say(f"share {r}: experts [{e_lo}, {e_lo + e_cnt})")
        loc = ref.local_expert_ids(fw["idx"], e_lo, e_cnt)
        c_r, o_r, d_r, s_r = ref.build_index(loc, e_cnt)
        i32 = lambda *shape: torch.empty(*shape, dtype=torch.int32, device=DEV)
        counts, offsets, dst_row, src_tok = i32(e_cnt), i32(e_cnt + 1), i32(T, k), i32(T * k)
        xp = torch.empty(T * k, h, dtype=torch.bfloat16, device=DEV)
        wsb = ops.moe_permute_local_workspace_size(T, e_cnt, k)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        ops.moe_permute_local(xd, MOE_BF16, idx, None, T, h, E, k, e_lo, e_cnt, counts, offsets, dst_row,
                              src_tok, xp, MOE_BF16, None, ws, wsb)
        torch.cuda.synchronize()
        rows = int(o_r[-1])
        np.testing.assert_array_equal(counts.cpu().numpy(), c_r)
        np.testing.assert_array_equal(offsets.cpu().numpy(), o_r)
        np.testing.assert_array_equal(dst_row.cpu().numpy(), d_r)
        np.testing.assert_array_equal(src_tok.cpu().numpy()[:rows], s_r[:rows])
        np.testing.assert_array_equal(host(xp)[:rows], f("x")[s_r[:rows]])
        # the share's experts and its partial output
        sl = slice(e_lo, e_lo + e_cnt)
        P = ops.PackedWeights(dev_tensor(inp["w1"][sl]), dev_tensor(inp["w3"][sl]), dev_tensor(inp["w2"][sl]),
                              MOE_BF16)
        yp = torch.empty(max(rows, 1), h, dtype=torch.float32, device=DEV)
        gwsb = ops.moe_grouped_workspace_size(max(rows, 1), h, hf, e_cnt, MOE_BF16)
        gws = torch.empty(gwsb, dtype=torch.uint8, device=DEV)
        if rows:
            ops.moe_grouped_swiglu_fwd(xp, None, P.struct, offsets, rows, None, yp, MOE_F32, gws, gwsb)
        part = torch.empty(T, h, dtype=torch.float32, device=DEV)
        ops.moe_combine(yp, MOE_F32, dst_row, w, T, h, k, part, MOE_F32)
        torch.cuda.synchronize()
        total += part.cpu().numpy()
    # expert outputs and partial sums in fp32: the plain bar
    check_close(total, fw["y"], 2e-2, None, None, "sum of the shares' partial outputs")
