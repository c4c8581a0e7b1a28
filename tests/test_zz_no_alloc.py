"""The allocation-free attention entry point (sb_op_attention_noalloc) against sb_op_attention with a
caller workspace, through the C ABI: two calls in a row, the second on a smaller batch."""
import os
import re

import numpy as np
import pytest
import torch

import selective_batching_amd as sb
from gpu_util import print_case
from synth import ModelDims, normal
from selective_batching_amd.runtime import make_dims, stream_handle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
M = ModelDims("noalloc", "llama", n_layers=1, H=1024, nq=8, nkv=2, d=128, F=512, V=64, max_pos=0)


def test_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "sb_ops.h")).read()
    m = re.search(r"#define SB_ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == sb.SB_ATTN_NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_batches_beyond_its_scratch():
    """A batch whose split partials exceed the static array is refused before any launch (no GPU needed:
    the metadata stays on the host and no kernel is reached)."""
    dims = make_dims(M, "bf16")
    batch = [(1, 4_000_000)]                        # 7813 units per K/V head, all left as partials
    kv = sb.sb_kv_create(4_000_008, 4_000_008, 1, M.nkv, M.d, sb.SB_BF16)
    nb = sb.sb_ragged_bytes(dims, 1, 1, 4_000_001)
    buf = np.zeros(nb // 4 + 16, np.int32)
    rg = sb.sb_ragged_build(dims, [1], [4_000_000], [0], None, buf.ctypes.data, None, buf.nbytes)
    assert rg.n_partials * 16 * (M.d + 2) * 4 > sb.SB_ATTN_NOALLOC_SCRATCH_BYTES
    with pytest.raises(sb.SBError) as e:
        sb.sb_op_attention_noalloc(dims, rg, kv, 0, 1 << 20, 1 << 20)
    assert e.value.status == sb.SB_ERR_WORKSPACE
    sb.sb_kv_destroy(kv)


def _attention_both_ways(kv, dims, batch, bases, seed, meta, staging):
    T = sum(n for n, _ in batch)
    rg = sb.sb_ragged_build(dims, [n for n, _ in batch], [c for _, c in batch], bases, None, staging.data_ptr(),
                            meta.data_ptr(), meta.numel(), stream_handle())
    qkv = torch.from_numpy(normal(seed, "noalloc.qkv", (T, M.qkv_out), dtype="bf16")).cuda().to(torch.bfloat16)
    o_ws = torch.full((T, M.nq * M.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    o_na = torch.full((T, M.nq * M.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(rg.n_partials, 1) * 16 * (M.d + 2) * 4, dtype=torch.uint8, device="cuda")
    s = stream_handle()
    sb.sb_op_attention(dims, rg, kv, 0, qkv.data_ptr(), o_ws.data_ptr(), ws.data_ptr(), ws.numel(), s)
    sb.sb_op_attention_noalloc(dims, rg, kv, 0, qkv.data_ptr(), o_na.data_ptr(), s)
    torch.cuda.synchronize()
    return rg, o_ws, o_na


@pytest.mark.gpu
def test_noalloc_attention_equals_workspace_attention():
    """Decodes over long histories (several 512-key units each, so split partials go through the scratch)
    plus a prompt chunk on top of cached tokens; then a second, smaller batch on the same array.  The
    outputs equal those of the workspace entry point bitwise (the same kernels in the same order)."""
    dims = make_dims(M, "bf16")
    batches = [[(1, 3000), (1, 1700), (1, 513), (1, 40), (37, 900), (1, 2600)],
               [(1, 1100), (5, 700)]]
    print_case("noalloc attention", batches)
    n_slots = 16384
    arena = sb.sb_kv_arena_slots(n_slots, 8)
    nb = sb.sb_kv_arena_bytes(arena, 1, M.nkv, M.d, sb.SB_BF16)
    ka = torch.empty(nb // 2, dtype=torch.bfloat16, device="cuda")
    va = torch.empty(nb // 2, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    ka.normal_(0.0, 1.0, generator=g)
    va.normal_(0.0, 1.0, generator=g)
    kv = sb.sb_kv_create(n_slots, arena, 1, M.nkv, M.d, sb.SB_BF16, ka.data_ptr(), va.data_ptr())
    try:
        mb = sb.sb_ragged_bytes(dims, 8, 64, n_slots)
        staging = torch.empty(mb, dtype=torch.uint8, pin_memory=True)
        meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
        n_parts = []
        for k, batch in enumerate(batches):
            rid0 = 100 * (k + 1)
            bases = [sb.sb_kv_reserve(kv, rid0 + i, n + c) for i, (n, c) in enumerate(batch)]
            rg, o_ws, o_na = _attention_both_ways(kv, dims, batch, bases, k, meta, staging)
            n_parts.append(rg.n_partials)
            assert rg.n_partials > 0
            a, b = o_ws.float().cpu().numpy(), o_na.float().cpu().numpy()
            assert np.all(np.isfinite(a))
            assert np.array_equal(a, b), f"call {k}: max |diff| {np.nanmax(np.abs(a - b))}"
            print(f"[case] call {k}: {rg.n_tokens} rows, {rg.n_partials} partials: bitwise equal", flush=True)
            for i in range(len(batch)):
                sb.sb_kv_free(kv, rid0 + i)
        assert n_parts[1] < n_parts[0]
    finally:
        sb.sb_kv_destroy(kv)
