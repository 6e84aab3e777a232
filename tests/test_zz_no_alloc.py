"""moe_permute_noalloc (the dispatch with its index scratch in a file-scope
device array, for callers that cannot allocate) against moe_permute with a
caller's workspace: counts, offsets, dst_row, src_tok and the copied rows
bit-exact, on two calls in a row, the second with a smaller input (the
array keeps the first call's contents), plus an FP8 dispatch; and sizes
beyond the scratch rejected before anything is written."""
import numpy as np
import pytest
import torch

import moe_synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from mixture_experts_layer_24_amd import ops
    from mixture_experts_layer_24_amd._lib import (MOE_BF16, MOE_ERR_WORKSPACE, MOE_FP8_E4M3, MOE_OK, lib)

DEV = "cuda"


def _buffers(T, E, k, h, dt):
    i32 = dict(dtype=torch.int32, device=DEV)
    return dict(counts=torch.full((E,), -3, **i32), offsets=torch.full((E + 1,), -3, **i32),
                dst_row=torch.full((T, k), -3, **i32), src_tok=torch.full((T * k,), -3, **i32),
                dst=torch.zeros(T * k, h, dtype=dt, device=DEV),
                scale=torch.zeros(T * k, dtype=torch.float32, device=DEV))


def _run_both(T, E, k, h, seed, fp8=False):
    print(f"no-alloc permute T={T} E={E} k={k} h={h} fp8={fp8}", flush=True)
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    idx[: T // 4] = np.arange(k, dtype=np.int32)             # one crowded expert block
    x = torch.from_numpy(moe_synth.f32_to_bf16_bits(rng.standard_normal((T, h)).astype(np.float32))
                         .view(np.int16)).to(DEV).view(torch.bfloat16)
    di = torch.from_numpy(idx).to(DEV)
    ddt, dcode = (torch.uint8, MOE_FP8_E4M3) if fp8 else (torch.bfloat16, MOE_BF16)
    a, b = _buffers(T, E, k, h, ddt), _buffers(T, E, k, h, ddt)
    wsb = ops.moe_permute_workspace_size(T, E, k)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    ops.moe_permute(x, MOE_BF16, di, None, T, h, E, k, a["counts"], a["offsets"], a["dst_row"], a["src_tok"],
                    a["dst"], dcode, a["scale"] if fp8 else None, ws, wsb)
    ops.moe_permute_noalloc(x, MOE_BF16, di, None, T, h, E, k, b["counts"], b["offsets"], b["dst_row"],
                            b["src_tok"], b["dst"], dcode, b["scale"] if fp8 else None)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key].view(torch.uint8) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.uint8) if b[key].dtype == torch.bfloat16 else b[key]), key
    assert int(b["counts"].sum()) == T * k


def test_noalloc_permute_matches_workspace_permute_twice():
    _run_both(3000, 64, 6, 128, 1)          # first call fills the scratch
    _run_both(500, 8, 2, 256, 2)            # a smaller input over the same scratch
    _run_both(300, 16, 1, 384, 3, fp8=True)


def test_noalloc_permute_rejects_sizes_beyond_its_scratch():
    L = lib()
    T, E, k, h = 262144 + 256, 256, 1, 8      # ceil(T / 256) * E * 4 bytes > 1 MiB
    i32 = dict(dtype=torch.int32, device=DEV)
    idx = torch.zeros(1, k, **i32)             # never read: the size check comes first
    counts = torch.full((E,), -3, **i32)
    buf = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    rc = L.moe_permute_noalloc(buf.data_ptr(), MOE_BF16, idx.data_ptr(), None, T, h, E, k, counts.data_ptr(),
                               counts.data_ptr(), idx.data_ptr(), idx.data_ptr(), buf.data_ptr(), MOE_BF16,
                               None, None)
    assert rc == MOE_ERR_WORKSPACE and b"scratch" in L.moe_last_error()
    torch.cuda.synchronize()
    assert (counts == -3).all()
    # the largest T that fits with E = 256 is accepted by the size check
    assert ops.moe_permute_workspace_size(262144, 256, 1) <= 1 << 20 < ops.moe_permute_workspace_size(T, E, k)
