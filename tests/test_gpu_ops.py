"""GPU parity of each step of the iteration (op-level C entry points) against the oracle."""
import os

import numpy as np
import pytest
import torch

import selective_batching_amd as sb
from gpu_util import TOL, assert_close_attention, assert_close_elem, assert_close_rms, dev, host, print_case
from oracle import model as OM
from synth import ModelDims, bf16_round, normal, random_ragged_batch, synthetic_kv
from selective_batching_amd.runtime import make_dims, stream_handle

pytestmark = pytest.mark.gpu

DT = {"fp32": sb.SB_F32, "bf16": sb.SB_BF16}


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------- GEMM
GEMM_SHAPES = [(1, 64, 64), (7, 192, 64), (100, 320, 256), (129, 256, 128), (300, 640, 512), (64, 1024, 256)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("epi", ["store", "bias", "gelu", "resid", "swiglu"])
def test_gemm_matches_oracle(dtype, M, N, K, epi):
    print_case("gemm", dtype, M, N, K, epi)
    seed = M * 7 + N * 3 + K
    A = normal(seed, "A", (M, K), dtype=dtype)
    Wrows = 2 * N if epi == "swiglu" else N
    W = normal(seed, "W", (Wrows, K), std=0.05, dtype=dtype)
    b = normal(seed, "b", (N,), std=0.5, dtype=dtype) if epi in ("bias", "gelu", "resid") else None
    x0 = normal(seed, "x0", (M, N)).astype(np.float64)
    lin = OM.linear(A, W[:N], b)
    if epi in ("store", "bias"):
        want, code = lin, sb.SB_EPI_STORE
    elif epi == "gelu":
        want, code = OM.gelu(lin), sb.SB_EPI_GELU
    elif epi == "resid":
        want, code = x0 + lin, sb.SB_EPI_RESID
    else:
        want, code = OM.silu(OM.linear(A, W[:N])) * OM.linear(A, W[N:]), sb.SB_EPI_SWIGLU
    dA, dW = dev(A, dtype), dev(W, dtype)
    db = dev(b, dtype) if b is not None else None
    if epi == "resid":
        out = torch.from_numpy(x0.astype(np.float32)).cuda()
    else:
        out = torch.zeros((M, N), dtype=dA.dtype, device="cuda")
    sb.sb_op_gemm(DT[dtype], code, M, N, K, dA.data_ptr(), K, dW.data_ptr(), K, db.data_ptr() if db is not None else None,
                  out.data_ptr(), N, 0, N if epi == "swiglu" else 0, stream_handle())
    _sync()
    if dtype == "bf16" and epi != "resid":
        assert_close_elem(host(out), want, dtype, f"gemm {dtype} {M}x{N}x{K} {epi}")      # one bf16 rounding
    else:
        assert_close_rms(host(out), want, TOL["fp32"], f"gemm {dtype} {M}x{N}x{K} {epi}")


def test_gemm_fp32_logits_out_and_ragged_rows():
    """fp32 output of a bf16 GEMM (LM-head form), M not a multiple of any tile."""
    M, N, K = 37, 4096 + 64, 256
    A = normal(1, "A", (M, K), dtype="bf16")
    W = normal(1, "W", (N, K), std=0.05, dtype="bf16")
    out = torch.full((M, N), -7.0, dtype=torch.float32, device="cuda")
    dA, dW = dev(A, "bf16"), dev(W, "bf16")
    sb.sb_op_gemm(sb.SB_BF16, sb.SB_EPI_STORE, M, N, K, dA.data_ptr(), K, dW.data_ptr(), K, None,
                  out.data_ptr(), N, 1, 0, stream_handle())
    _sync()
    assert_close_rms(host(out), OM.linear(A, W), 1e-5, "bf16 gemm fp32 out")


# ---------------------------------------------------------------- norms
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("H,rows", [(64, 5), (256, 5), (2048, 5), (4096, 5), (12288, 5), (2048, 1031), (4096, 1031),
                                    (1028, 1500), (4096, 3741)])
def test_norm_matches_oracle(dtype, kind, H, rows):
    """Every launch shape: a workgroup per row (few rows, wide rows), a wave per row, and waves streaming
    several rows each (1028: a partial last group of pieces per lane; 3741: the 8B-shaped batch)."""
    print_case("norm", dtype, kind, H, rows)
    x = normal(H, "x", (rows + 2, H), std=2.0, mean=0.3)
    g = normal(H, "g", (H,), std=0.1, mean=1.0, dtype=dtype)
    b = normal(H, "b", (H,), std=0.1, dtype=dtype) if kind == 0 else None
    row_map = np.array([6, 0, 3, 3, 1], np.int32) if rows == 5 else \
        np.random.default_rng(H).integers(0, rows + 2, rows).astype(np.int32)
    out = torch.zeros((rows, H), dtype={"fp32": torch.float32, "bf16": torch.bfloat16}[dtype], device="cuda")
    dx = torch.from_numpy(x).cuda()
    dmap = torch.from_numpy(row_map).cuda()
    dg, dbb = dev(g, dtype), (dev(b, dtype) if b is not None else None)
    sb.sb_op_norm(DT[dtype], kind, rows, H, dx.data_ptr(), dmap.data_ptr(), dg.data_ptr(),
                  dbb.data_ptr() if dbb is not None else None, 1e-5, out.data_ptr(), stream_handle())
    _sync()
    xs = x[row_map].astype(np.float64)
    want = OM.layer_norm(xs, g, b, 1e-5) if kind == 0 else OM.rms_norm(xs, g, 1e-5)
    assert_close_elem(host(out), want, dtype, f"norm {dtype} kind {kind} H {H}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("H", [1028, 2048, 4096])
def test_norm_independent_of_row_count(dtype, kind, H):
    """A row's normalised values do not depend on how many rows are normalised with it: 7 rows alone
    (a workgroup per row) and the same rows among 1500 (waves streaming rows) give the same bits."""
    print_case("norm row-count invariance", dtype, kind, H)
    rows = 1500
    x = normal(H + 1, "x", (rows, H), std=2.0, mean=0.3)
    g = normal(H + 1, "g", (H,), std=0.1, mean=1.0, dtype=dtype)
    b = normal(H + 1, "b", (H,), std=0.1, dtype=dtype) if kind == 0 else None
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]
    dx = torch.from_numpy(x).cuda()
    dg, dbb = dev(g, dtype), (dev(b, dtype) if b is not None else None)
    pick = np.array([1499, 0, 700, 3, 3, 1024, 58], np.int32)
    outs = []
    for n, row_map in ((rows, None), (len(pick), pick)):
        out = torch.zeros((n, H), dtype=tdt, device="cuda")
        dmap = torch.from_numpy(row_map).cuda() if row_map is not None else None
        sb.sb_op_norm(DT[dtype], kind, n, H, dx.data_ptr(), dmap.data_ptr() if dmap is not None else None,
                      dg.data_ptr(), dbb.data_ptr() if dbb is not None else None, 1e-5, out.data_ptr(),
                      stream_handle())
        _sync()
        outs.append(out.view(torch.int32 if dtype == "fp32" else torch.int16).cpu())
    assert torch.equal(outs[0][torch.from_numpy(pick).long()], outs[1])


# ---------------------------------------------------------------- argmax
def test_argmax_ties_and_random():
    V = 128256
    x = normal(0, "logits", (6, V)).astype(np.float32)
    x[1, 17] = x[1, 900] = x[1, 50000] = 100.0          # tie: lowest index wins
    x[2, :] = 0.0
    x[3, V - 1] = 1e9
    d = torch.from_numpy(x).cuda()
    out = torch.zeros(6, dtype=torch.int32, device="cuda")
    sb.sb_op_argmax(6, V, d.data_ptr(), out.data_ptr(), stream_handle())
    _sync()
    got = out.cpu().numpy()
    assert list(got) == [OM.greedy(r) for r in x]
    assert got[1] == 17 and got[2] == 0 and got[3] == V - 1


# ---------------------------------------------------------------- attention (+ RoPE / K/V append)
def _attention_case(m: ModelDims, dtype, batch, seed, rope_check=False):
    """Random q/k/v for the new tokens, synthetic history in the K/V manager; GPU vs oracle."""
    print_case("attention", m.name, dtype, batch, seed)
    dims = make_dims(m, dtype)
    G = m.nq // m.nkv
    n_slots = sum(n + c for n, c in batch) + 64
    arena = sb.sb_kv_arena_slots(n_slots, len(batch))
    nbytes = sb.sb_kv_arena_bytes(arena, 1, m.nkv, m.d, DT[dtype])
    ka = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")     # non-zero garbage outside writes
    va = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
    kv = sb.sb_kv_create(n_slots, arena, 1, m.nkv, m.d, DT[dtype], ka.data_ptr(), va.data_ptr())
    try:
        bases, hist, keep = [], [], []
        for i, (n, c) in enumerate(batch):
            base = sb.sb_kv_reserve(kv, i, n + c)
            bases.append(base)
            hk, hv = synthetic_kv(seed, f"h{i}", c, m.nkv, m.d, 1.0, dtype)
            hist.append((hk, hv))
            if c:
                slots = torch.arange(base, base + c, dtype=torch.int32, device="cuda")
                dk, dv = dev(hk, dtype), dev(hv, dtype)
                keep += [slots, dk, dv]
                sb.sb_kv_write(kv, 0, c, slots.data_ptr(), dk.data_ptr(), dv.data_ptr(), stream_handle())
        T = sum(n for n, _ in batch)
        qkv = normal(seed, "qkv", (T, m.qkv_out), dtype=dtype)
        nbytes_meta = sb.sb_ragged_bytes(dims, len(batch), T, n_slots)
        staging = torch.empty(nbytes_meta, dtype=torch.uint8, pin_memory=True)
        meta = torch.empty(nbytes_meta, dtype=torch.uint8, device="cuda")
        rg = sb.sb_ragged_build(dims, [n for n, _ in batch], [c for _, c in batch], bases, None, staging.data_ptr(),
                                meta.data_ptr(), nbytes_meta, stream_handle())
        dqkv = dev(qkv, dtype)
        sb.sb_op_rope_append(dims, rg, kv, 0, dqkv.data_ptr(), stream_handle())
        o = torch.zeros((T, m.nq * m.d), dtype=dqkv.dtype, device="cuda")
        ws = torch.empty(max(rg.n_partials, 1) * 16 * (m.d + 2) * 4, dtype=torch.uint8, device="cuda")
        sb.sb_op_attention(dims, rg, kv, 0, dqkv.data_ptr(), o.data_ptr(), ws.data_ptr(), ws.numel(), stream_handle())
        # the rows just appended, read back through the manager (rotated k for Llama)
        new_slots = np.concatenate([np.arange(bases[i] + c, bases[i] + c + n)
                                    for i, (n, c) in enumerate(batch)]).astype(np.int32)
        dnew = torch.from_numpy(new_slots).cuda()
        kk_new = torch.zeros((T, m.nkv, m.d), dtype=dqkv.dtype, device="cuda")
        vv_new = torch.zeros_like(kk_new)
        sb.sb_kv_read(kv, 0, T, dnew.data_ptr(), kk_new.data_ptr(), vv_new.data_ptr(), stream_handle())
        _sync()
        got = host(o)
        got_qkv = host(dqkv)
        want = np.zeros_like(got)
        want_abs = np.zeros_like(got)
        t0 = 0
        nq_d, nkv_d = m.nq * m.d, m.nkv * m.d
        for i, (n, c) in enumerate(batch):
            rows = slice(t0, t0 + n)
            q = qkv[rows, :nq_d].reshape(n, m.nq, m.d).astype(np.float64)
            k = qkv[rows, nq_d:nq_d + nkv_d].reshape(n, m.nkv, m.d).astype(np.float64)
            v = qkv[rows, nq_d + nkv_d:].reshape(n, m.nkv, m.d).astype(np.float64)
            if m.arch == "llama":
                pos = c + np.arange(n)
                q, k = OM.rope(q, pos, m.rope_theta), OM.rope(k, pos, m.rope_theta)
                assert_close_elem(got_qkv[rows, :nq_d], q.reshape(n, nq_d), dtype, "rope q")
                assert_close_elem(host(kk_new[rows]).reshape(n, nkv_d), k.reshape(n, nkv_d), dtype, "rope k")
                # attention is checked on the rotated q, k exactly as stored on the GPU
                q = got_qkv[rows, :nq_d].reshape(n, m.nq, m.d)
                k = host(kk_new[rows])
            K = np.concatenate([hist[i][0].astype(np.float64), k], axis=0)
            V = np.concatenate([hist[i][1].astype(np.float64), v], axis=0)
            want[rows] = OM.attention(q, K, V, c, G).reshape(n, nq_d)
            want_abs[rows] = OM.attention(q, K, np.abs(V), c, G).reshape(n, nq_d)
            t0 += n
        # one rounding of the exact attention of the stored q, k, v (fp32: a few fp32 operations; bf16: plus
        # the probabilities' 16-bit hi + lo representation)
        assert_close_attention(got, want, want_abs, dtype, f"attention {m.name} {dtype}")
        # the appended rows landed in their slots (V is copied as is; K too unless rotated)
        np.testing.assert_array_equal(host(vv_new).reshape(T, -1), qkv[:, nq_d + nkv_d:])
        if m.arch == "gpt":
            np.testing.assert_array_equal(host(kk_new).reshape(T, -1), qkv[:, nq_d:nq_d + nkv_d])
    finally:
        sb.sb_kv_destroy(kv)


TINY_F32 = ModelDims("attn-f32", "gpt", 1, H=64, nq=4, nkv=4, d=16, F=64, V=0)
MINI_ATT = ModelDims("attn-mini", "gpt", 1, H=256, nq=8, nkv=8, d=32, F=64, V=0)
GQA_BF16 = ModelDims("attn-gqa", "llama", 1, H=1024, nq=8, nkv=2, d=128, F=64, V=0, rope_theta=500000.0)
GQA_F32 = ModelDims("attn-gqa32", "llama", 1, H=512, nq=8, nkv=2, d=64, F=64, V=0, rope_theta=10000.0)
GQA64_BF16 = ModelDims("attn-gqa64", "llama", 1, H=512, nq=8, nkv=2, d=64, F=64, V=0, rope_theta=10000.0)


@pytest.mark.parametrize("m,dtype", [(TINY_F32, "fp32"), (MINI_ATT, "bf16"), (MINI_ATT, "fp32"), (GQA_BF16, "bf16"),
                                     (GQA_F32, "fp32"), (GQA64_BF16, "bf16")])
def test_attention_figure5_and_exercise4(m, dtype):
    _attention_case(m, dtype, [(1, 3), (1, 1), (2, 0), (3, 0)], 1, rope_check=True)
    _attention_case(m, dtype, [(37, 0), (9, 0), (1, 120), (1, 15), (1, 64)], 2)


@pytest.mark.parametrize("m,dtype", [(MINI_ATT, "bf16"), (GQA_BF16, "bf16"), (GQA_F32, "fp32"), (TINY_F32, "fp32"),
                                     (GQA64_BF16, "bf16")])
@pytest.mark.parametrize("seed", range(3))
def test_attention_random_ragged(m, dtype, seed):
    batch = random_ragged_batch(seed, 7, 1500, 90)     # long histories -> split items; big prefills -> row tiles
    _attention_case(m, dtype, batch, seed + 10)


# new tokens that start, end and straddle 8-slot blocks of the blocked V layout: decodes sharing a block
# with their history, prompts filling whole blocks, runs crossing one or two block edges
BLOCK_EDGES = [(1, 7), (1, 8), (1, 15), (8, 0), (9, 7), (17, 3), (3, 5), (16, 16), (1, 0), (7, 1), (24, 8)]


@pytest.mark.parametrize("m,dtype", [(GQA_BF16, "bf16"), (GQA_F32, "fp32"), (TINY_F32, "fp32")])
def test_attention_append_block_edges(m, dtype):
    _attention_case(m, dtype, BLOCK_EDGES, 21, rope_check=m.arch == "llama")


@pytest.mark.parametrize("m,dtype", [(GQA_BF16, "bf16"), (TINY_F32, "fp32")])
def test_append_writes_only_its_slots(m, dtype):
    """RoPE/append writes each new token's K and V at its own slot and nowhere else: every other slot of
    the arenas (history, reserved but unused, unreserved) keeps its bytes."""
    print_case("append slots", m.name, dtype)
    dims = make_dims(m, dtype)
    batch = BLOCK_EDGES
    n_slots = sum(n + c + 9 for n, c in batch) + 64
    arena = sb.sb_kv_arena_slots(n_slots, len(batch))
    nbytes = sb.sb_kv_arena_bytes(arena, 1, m.nkv, m.d, DT[dtype])
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    ka = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    va = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    ka0, va0 = ka.cpu(), va.cpu()
    kv = sb.sb_kv_create(n_slots, arena, 1, m.nkv, m.d, DT[dtype], ka.data_ptr(), va.data_ptr())
    try:
        bases = [sb.sb_kv_reserve(kv, i, n + c + 9) for i, (n, c) in enumerate(batch)]   # 9 spare slots each
        T = sum(n for n, _ in batch)
        qkv = normal(9, "qkv", (T, m.qkv_out), dtype=dtype)
        mb = sb.sb_ragged_bytes(dims, len(batch), T, n_slots)
        staging = torch.empty(mb, dtype=torch.uint8, pin_memory=True)
        meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
        rg = sb.sb_ragged_build(dims, [n for n, _ in batch], [c for _, c in batch], bases, None, staging.data_ptr(),
                                meta.data_ptr(), mb, stream_handle())
        dqkv = dev(qkv, dtype)
        sb.sb_op_rope_append(dims, rg, kv, 0, dqkv.data_ptr(), stream_handle())
        _sync()
        new = set(b + c + j for b, (n, c) in zip(bases, batch) for j in range(n))
        es = 2 if dtype == "bf16" else 4
        row = m.d * es                                       # bytes of one slot of one K/V head
        k1, v1 = ka.cpu(), va.cpu()
        # K: [kv head][slot][d]; V: [kv head][slot / 8][d][slot % 8]
        kmask = np.zeros(nbytes, bool)
        vmask = np.zeros(nbytes, bool)
        for h in range(m.nkv):
            for s in new:
                kmask[(h * arena + s) * row:(h * arena + s + 1) * row] = True
                blk = (h * arena * m.d + (s // 8) * m.d * 8) * es
                for e in range(m.d):
                    o = blk + (e * 8 + s % 8) * es
                    vmask[o:o + es] = True
        kchg = (k1.numpy() != ka0.numpy())
        vchg = (v1.numpy() != va0.numpy())
        assert not np.any(kchg & ~kmask), "K bytes changed outside the new tokens' slots"
        assert not np.any(vchg & ~vmask), "V bytes changed outside the new tokens' slots"
    finally:
        sb.sb_kv_destroy(kv)


@pytest.mark.parametrize("m", [GQA_BF16, GQA64_BF16, ModelDims("attn-gqa-d32", "llama", 1, H=256, nq=8, nkv=2, d=32,
                                                              F=64, V=0, rope_theta=10000.0)])
def test_attention_prefill_tile_shape_invariant(m):
    """A prompt's attention alone (few row tiles: 64-row tiles, 16 real rows per wave) and among 32 other
    prompts (over 1024 tiles of 64 rows: 128-row tiles, 32 real rows per wave) gives the same bits: a row's
    arithmetic does not depend on the tile it falls in."""
    dims = make_dims(m, "bf16")
    target = (300, 17)
    others = [(256, 0)] * 32
    print_case("prefill tile shape invariance", m.name)
    outs = []
    for batch in ([target], others + [target]):
        n_slots = sum(n + c for n, c in batch) + 8 * len(batch)
        arena = sb.sb_kv_arena_slots(n_slots, len(batch))
        nbytes = sb.sb_kv_arena_bytes(arena, 1, m.nkv, m.d, sb.SB_BF16)
        ka = torch.zeros(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        va = torch.zeros(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        kv = sb.sb_kv_create(n_slots, arena, 1, m.nkv, m.d, sb.SB_BF16, ka.data_ptr(), va.data_ptr())
        try:
            bases = [sb.sb_kv_reserve(kv, i, n + c) for i, (n, c) in enumerate(batch)]
            ti = len(batch) - 1                              # the target is the last request
            hk, hv = synthetic_kv(5, "target", target[1], m.nkv, m.d, 1.0, "bf16")
            slots = torch.arange(bases[ti], bases[ti] + target[1], dtype=torch.int32, device="cuda")
            dk, dv = dev(hk, "bf16"), dev(hv, "bf16")
            sb.sb_kv_write(kv, 0, target[1], slots.data_ptr(), dk.data_ptr(), dv.data_ptr(), stream_handle())
            T = sum(n for n, _ in batch)
            qkv = np.concatenate([normal(6 + i, "qkv", (n, m.qkv_out), dtype="bf16") for i, (n, _) in enumerate(batch[:-1])]
                                 + [normal(99, "qkv-target", (target[0], m.qkv_out), dtype="bf16")])
            mb = sb.sb_ragged_bytes(dims, len(batch), T, n_slots)
            staging = torch.empty(mb, dtype=torch.uint8, pin_memory=True)
            meta = torch.empty(mb, dtype=torch.uint8, device="cuda")
            rg = sb.sb_ragged_build(dims, [n for n, _ in batch], [c for _, c in batch], bases, None,
                                    staging.data_ptr(), meta.data_ptr(), mb, stream_handle())
            dqkv = dev(qkv, "bf16")
            sb.sb_op_rope_append(dims, rg, kv, 0, dqkv.data_ptr(), stream_handle())
            o = torch.zeros((T, m.nq * m.d), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(max(rg.n_partials, 1) * 16 * (m.d + 2) * 4, dtype=torch.uint8, device="cuda")
            sb.sb_op_attention(dims, rg, kv, 0, dqkv.data_ptr(), o.data_ptr(), ws.data_ptr(), ws.numel(),
                               stream_handle())
            _sync()
            outs.append(o[T - target[0]:].view(torch.int16).cpu())
        finally:
            sb.sb_kv_destroy(kv)
    assert torch.equal(outs[0], outs[1])


def test_attention_decode_only():
    _attention_case(MINI_ATT, "bf16", [(1, 100), (1, 17), (1, 256), (1, 31), (1, 32)], 7)
    _attention_case(MINI_ATT, "fp32", [(1, 100), (1, 17), (1, 256), (1, 31), (1, 32)], 7)
    _attention_case(GQA_BF16, "bf16", [(1, 100), (1, 17), (1, 256), (1, 31), (1, 32)], 8)


def test_attention_edge_cases():
    _attention_case(GQA_BF16, "bf16", [(1, 0)], 3)                  # one token, no history: o = v
    _attention_case(GQA_BF16, "bf16", [(1, 2047)], 4)               # single long decode
    _attention_case(GQA_BF16, "bf16", [(64, 0), (65, 0), (17, 511)], 5)   # tile boundaries
    _attention_case(MINI_ATT, "bf16", [(16, 512), (1, 512), (1, 513)], 6)  # split boundaries


N_GEMM_CFGS = 28  # register-staged 128x128, 256x256 (4 and 8 waves), 256x128, 128x256; DMA-fed: 4 with BK 32, 2 with BK 64, 2 spread, 256x192 + 192x256 spread, skinny 64x32 / 64x16 / 64x64 with deep K pipelines, 256x384 spread; register rings 64x32, 64x64, 32x32, 32x64, 96x64, 96x96, 128x128 (128-deep K steps, or 64-deep when K % 128 != 0); DMA-fed 224x384 spread (76 copies per stage, split unevenly over 8 waves); register ring 64x128


@pytest.mark.parametrize("cfg", range(N_GEMM_CFGS))
@pytest.mark.parametrize("epi", ["bias", "gelu", "resid", "swiglu"])
@pytest.mark.parametrize("K", [512, 64, 192, 256, 384])
def test_gemm_every_tile_config(cfg, epi, K, monkeypatch):
    """Each bf16 tile configuration (forced) on a ragged shape: M and N not multiples of the tile;
    K = 64 and 192 leave fewer K tiles than LDS stages / a partial ring trip (64-deep ring steps);
    K = 256 and 384 leave two and three of the rings' four 128-deep steps in flight."""
    monkeypatch.setenv("SB_GEMM_CFG", str(cfg))
    M, N = 300, 640
    print_case("gemm cfg", cfg, epi, M, N, K)
    A = normal(cfg, "A", (M, K), dtype="bf16")
    W = normal(cfg, "W", (2 * N if epi == "swiglu" else N, K), std=0.05, dtype="bf16")
    b = normal(cfg, "b", (N,), std=0.5, dtype="bf16")
    x0 = normal(cfg, "x0", (M, N)).astype(np.float64)
    code = {"bias": sb.SB_EPI_STORE, "gelu": sb.SB_EPI_GELU, "resid": sb.SB_EPI_RESID, "swiglu": sb.SB_EPI_SWIGLU}[epi]
    dA, dW, db = dev(A, "bf16"), dev(W, "bf16"), dev(b, "bf16")
    out = torch.from_numpy(x0.astype(np.float32)).cuda() if epi == "resid" else \
        torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    bias = None if epi == "swiglu" else db.data_ptr()
    sb.sb_op_gemm(sb.SB_BF16, code, M, N, K, dA.data_ptr(), K, dW.data_ptr(), K, bias, out.data_ptr(), N, 0,
                  N if epi == "swiglu" else 0, stream_handle())
    _sync()
    lin = OM.linear(A, W[:N], None if epi == "swiglu" else b)
    if epi == "bias":
        assert_close_elem(host(out), lin, "bf16", f"cfg {cfg} bias")
    elif epi == "gelu":
        assert_close_elem(host(out), OM.gelu(lin), "bf16", f"cfg {cfg} gelu")
    elif epi == "resid":
        assert_close_rms(host(out), x0 + lin, TOL["fp32"], f"cfg {cfg} resid")
    else:
        assert_close_elem(host(out), OM.silu(OM.linear(A, W[:N])) * OM.linear(A, W[N:]), "bf16", f"cfg {cfg} swiglu")


@pytest.mark.parametrize("cfg", range(N_GEMM_CFGS))
@pytest.mark.parametrize("epi", ["resid", "swiglu"])
@pytest.mark.parametrize("M", [1, 33])
def test_gemm_every_tile_config_few_rows(cfg, epi, M, monkeypatch):
    """Each configuration (forced) with fewer rows than its tile: one row, or a ragged 33 (row clamping,
    masked stores); K = 192 (three 64-deep tiles, fewer than the deeper rings)."""
    monkeypatch.setenv("SB_GEMM_CFG", str(cfg))
    N, K = 96, 192
    print_case("gemm cfg few rows", cfg, epi, M, N, K)
    A = normal(cfg + 50, "A", (M, K), dtype="bf16")
    W = normal(cfg + 50, "W", (2 * N if epi == "swiglu" else N, K), std=0.05, dtype="bf16")
    x0 = normal(cfg + 50, "x0", (M, N)).astype(np.float64)
    dA, dW = dev(A, "bf16"), dev(W, "bf16")
    if epi == "resid":
        out = torch.from_numpy(x0.astype(np.float32)).cuda()
        sb.sb_op_gemm(sb.SB_BF16, sb.SB_EPI_RESID, M, N, K, dA.data_ptr(), K, dW.data_ptr(), K, None, out.data_ptr(),
                      N, 0, 0, stream_handle())
        _sync()
        assert_close_rms(host(out), x0 + OM.linear(A, W), TOL["fp32"], f"cfg {cfg} resid M {M}")
    else:
        out = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
        sb.sb_op_gemm(sb.SB_BF16, sb.SB_EPI_SWIGLU, M, N, K, dA.data_ptr(), K, dW.data_ptr(), K, None, out.data_ptr(),
                      N, 0, N, stream_handle())
        _sync()
        assert_close_elem(host(out), OM.silu(OM.linear(A, W[:N])) * OM.linear(A, W[N:]), "bf16",
                          f"cfg {cfg} swiglu M {M}")


@pytest.mark.parametrize("epi", ["bias", "swiglu"])
@pytest.mark.parametrize("M", [300, 33])
@pytest.mark.parametrize("K", [512, 192])
def test_gemm_configs_bitwise_identical(epi, M, K, monkeypatch):
    """Every tile configuration gives the same bits: each output sums K in 32-wide MFMA steps in
    ascending order whatever the tile, so the launcher's choice (which depends on M, i.e. on the
    batch) never changes a result.  K = 192 takes the register rings' 64-deep steps, K = 512 their
    128-deep ones."""
    N = 640
    A = normal(7, "A", (M, K), dtype="bf16")
    W = normal(7, "W", (2 * N if epi == "swiglu" else N, K), std=0.05, dtype="bf16")
    b = normal(7, "b", (N,), std=0.5, dtype="bf16")
    code = sb.SB_EPI_SWIGLU if epi == "swiglu" else sb.SB_EPI_STORE
    dA, dW, db = dev(A, "bf16"), dev(W, "bf16"), dev(b, "bf16")
    outs = []
    for cfg in range(N_GEMM_CFGS):
        monkeypatch.setenv("SB_GEMM_CFG", str(cfg))
        out = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
        sb.sb_op_gemm(sb.SB_BF16, code, M, N, K, dA.data_ptr(), K, dW.data_ptr(), K,
                      None if epi == "swiglu" else db.data_ptr(), out.data_ptr(), N, 0, N if epi == "swiglu" else 0,
                      stream_handle())
        _sync()
        outs.append(out.view(torch.int16).cpu())
    for cfg in range(1, N_GEMM_CFGS):
        assert torch.equal(outs[cfg], outs[0]), f"cfg {cfg} differs from cfg 0"


# indices of register-ring tiles in the launcher's configuration list
CFG_RING_32x32, CFG_RING_96x64, CFG_RING_128x128, CFG_RING_64x128 = 21, 23, 25, 27


@pytest.mark.parametrize("cfg", [CFG_RING_64x128, CFG_RING_128x128, CFG_RING_96x64])
@pytest.mark.parametrize("M", [64, 200])
@pytest.mark.parametrize("K", [4096, 14336])
@pytest.mark.parametrize("epi", ["swiglu", "resid"])
def test_gemm_ring_tiles_at_model_k(cfg, M, K, epi, monkeypatch):
    """The register-ring tiles the small-problem picker takes at decode and mid sizes, at the 8B-shaped model's
    own K (4096: QKV, attention-out, FFN1, LM head; 14336: FFN2), i.e. over 32 or 112 of their 128-deep K steps:
    element-wise against the oracle, and bitwise equal to the 32 x 32 ring with its 256-deep steps (one MFMA
    chain per output over ascending K in both)."""
    N = 512
    print_case("gemm ring at model K", cfg, M, K, epi)
    A = normal(cfg + M, "A", (M, K), dtype="bf16")
    W = normal(cfg + M, "W", (2 * N if epi == "swiglu" else N, K), std=0.02, dtype="bf16")
    x0 = normal(cfg + M, "x0", (M, N)).astype(np.float64)
    dA, dW = dev(A, "bf16"), dev(W, "bf16")
    code = sb.SB_EPI_SWIGLU if epi == "swiglu" else sb.SB_EPI_RESID

    def run(c):
        monkeypatch.setenv("SB_GEMM_CFG", str(c))
        out = torch.from_numpy(x0.astype(np.float32)).cuda() if epi == "resid" else \
            torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
        sb.sb_op_gemm(sb.SB_BF16, code, M, N, K, dA.data_ptr(), K, dW.data_ptr(), K, None, out.data_ptr(), N, 0,
                      N if epi == "swiglu" else 0, stream_handle())
        _sync()
        return out

    got, ref = run(cfg), run(CFG_RING_32x32)
    view = torch.int32 if epi == "resid" else torch.int16
    assert torch.equal(got.view(view).cpu(), ref.view(view).cpu()), f"cfg {cfg} differs from the 32 x 32 ring"
    if epi == "resid":
        assert_close_rms(host(got), x0 + OM.linear(A, W), TOL["fp32"], f"cfg {cfg} resid M {M} K {K}")
    else:
        assert_close_elem(host(got), OM.silu(OM.linear(A, W[:N])) * OM.linear(A, W[N:]), "bf16",
                          f"cfg {cfg} swiglu M {M} K {K}")


def test_attention_unit_merge_is_batch_invariant():
    """A request's attention output does not depend on the batch around it.  Alone, its 512-key units are
    spread over several workgroups and merged by the combine step; among 400 long requests one workgroup
    runs all of its units and merges them itself.  Both must give the same bits (and match the oracle)."""
    m = GQA_BF16
    dims = make_dims(m, "bf16")
    G = m.nq // m.nkv
    batch = [(1, 1500 + (i % 7) * 37) for i in range(400)]
    print_case("attention batch invariance", m.name, len(batch))
    n_slots = sum(n + c for n, c in batch) + 8 * len(batch)
    arena = sb.sb_kv_arena_slots(n_slots, len(batch))
    nbytes = sb.sb_kv_arena_bytes(arena, 1, m.nkv, m.d, sb.SB_BF16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    ka = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
    va = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_(generator=gen)
    kv = sb.sb_kv_create(n_slots, arena, 1, m.nkv, m.d, sb.SB_BF16, ka.data_ptr(), va.data_ptr())
    try:
        bases = [sb.sb_kv_reserve(kv, i, n + c) for i, (n, c) in enumerate(batch)]
        qkv_all = dev(normal(12, "qkv", (len(batch), m.qkv_out), dtype="bf16"), "bf16")

        def run(idx):
            sub = [batch[i] for i in idx]
            T = len(idx)
            nb = sb.sb_ragged_bytes(dims, T, T, n_slots)
            staging = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
            meta = torch.empty(nb, dtype=torch.uint8, device="cuda")
            rg = sb.sb_ragged_build(dims, [n for n, _ in sub], [c for _, c in sub], [bases[i] for i in idx], None,
                                    staging.data_ptr(), meta.data_ptr(), nb, stream_handle())
            qkv = qkv_all[list(idx)].contiguous()
            o = torch.zeros((T, m.nq * m.d), dtype=torch.bfloat16, device="cuda")
            ws = torch.empty(max(rg.n_partials, 1) * 16 * (m.d + 2) * 4, dtype=torch.uint8, device="cuda")
            sb.sb_op_attention(dims, rg, kv, 0, qkv.data_ptr(), o.data_ptr(), ws.data_ptr(), ws.numel(),
                               stream_handle())
            _sync()
            return o, rg.n_groups

        o_big, groups_big = run(range(len(batch)))
        for r in (0, 3, 6):
            o_one, groups_one = run([r])
            assert groups_one == m.nkv                 # alone: split over workgroups, combined
            assert torch.equal(o_one[0].view(torch.int16), o_big[r].view(torch.int16)), f"request {r}"
        assert groups_big < m.nkv * len(batch)          # in the big batch most requests merge in one workgroup
        # and the result is the attention of the stored q, K, V
        n, c = batch[0]
        slots = torch.arange(bases[0], bases[0] + c + n, dtype=torch.int32, device="cuda")
        kk = torch.zeros((c + n, m.nkv, m.d), dtype=torch.bfloat16, device="cuda")
        vv = torch.zeros_like(kk)
        sb.sb_kv_read(kv, 0, c + n, slots.data_ptr(), kk.data_ptr(), vv.data_ptr(), stream_handle())
        _sync()
        q = host(qkv_all[0:1, :m.nq * m.d]).reshape(1, m.nq, m.d)
        want = OM.attention(q, host(kk), host(vv), c, G).reshape(1, -1)
        want_abs = OM.attention(q, host(kk), np.abs(host(vv)), c, G).reshape(1, -1)
        assert_close_attention(host(o_big[0:1]), want, want_abs, "bf16", "attention of a merged request")
    finally:
        sb.sb_kv_destroy(kv)


def test_package_imported_before_torch():
    """A fresh process that imports the package before torch still runs the library on the device
    (the package loads torch's HIP runtime before libsb.so, so there is one runtime)."""
    import subprocess
    import sys
    code = ("import selective_batching_amd as sb\n"
            "import torch\n"
            "x = torch.zeros(2, 300, device='cuda'); x[0, 7] = 1.0; x[1, 299] = 2.0\n"
            "out = torch.full((2,), -1, dtype=torch.int32, device='cuda')\n"
            "sb.sb_op_argmax(2, 300, x.data_ptr(), out.data_ptr(), torch.cuda.current_stream().cuda_stream)\n"
            "torch.cuda.synchronize()\n"
            "print(out.tolist())\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "[7, 299]"
