"""GPU parity of dwconv1d_stream_fwd (through the C ABI) against the CPU
oracle, and against the whole-sequence causal conv on the GPU."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import TOL_BF16, TOL_F32, assert_exact_zero, assert_parity, say, time_mask

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def lib():
    import conv_subsampling_amd as dw
    return dw


def make(B, Tc, C, K, dtype=torch.float32, seed=0, lens=None):
    tag = f"t1s/{B}/{Tc}/{C}/{K}/{seed}"
    x = datagen.normal((B, Tc, C), 1.0, tag + "/x", device=DEV).to(dtype)
    w = datagen.normal((K, C), 1.0 / K, tag + "/w", device=DEV).to(dtype)
    b = datagen.normal((C,), 0.1, tag + "/b", device=DEV).to(dtype)
    cache = datagen.normal((B, K - 1, C), 1.0, tag + "/cache", device=DEV).to(dtype)
    if lens is None:
        lens = datagen.int_uniform(B, -1, Tc + 1, tag + "/len")
    return x, w, b, cache, torch.as_tensor(lens, dtype=torch.int32).to(DEV)


def check(x, w, b, cache, L, what):
    B, Tc, C = x.shape
    say(f"dwconv1d_stream {what}: B={B} Tc={Tc} C={C} K={w.shape[0]} dtype={x.dtype} lengths={L.tolist()[:8]}")
    y, c2 = lib().dwconv1d_stream_fwd(x, w, b, L, cache)
    torch.cuda.synchronize()
    ry, rc = oracle.dwconv1d_stream_fwd(x, w, b, L, cache)
    tol = TOL_BF16 if x.dtype == torch.bfloat16 else TOL_F32
    assert_parity(y, ry, tol, what)
    assert np.array_equal(c2.float().cpu().numpy().astype(np.float64), rc), f"{what}: cache differs"
    assert_exact_zero(y, time_mask(L, B, Tc)[:, :, None], what)
    return y, c2


GRID = [
    # (B, Tc, C, K)
    (1, 1, 4, 3), (3, 1, 8, 9), (2, 2, 4, 5), (3, 7, 3, 4), (2, 50, 8, 15), (3, 5, 200, 9), (2, 17, 256, 3),
    (2, 13, 6, 1), (2, 9, 12, 2), (2, 20, 64, 7), (2, 40, 130, 31), (1, 100, 1, 9), (4, 8, 1024, 9),
    # the persistent form (16-byte lanes, chunks of at most 8 frames, 32 or more channel
    # groups): more streams than workgroups, a partial second slab, K = 15, one-frame chunks
    (1200, 8, 256, 9), (700, 3, 384, 4), (2100, 1, 512, 5), (600, 8, 256, 15), (5, 6, 1024, 3),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,Tc,C,K", GRID)
def test_grid(B, Tc, C, K, dtype):
    x, w, b, cache, L = make(B, Tc, C, K, dtype)
    check(x, w, b, cache, L, "grid")


@pytest.mark.parametrize("C", [64, 256])
@pytest.mark.parametrize("K", [3, 9, 15, 31])
def test_chunks_equal_the_whole_causal_conv_bitwise(K, C):
    """Streaming a sequence chunk by chunk (ping-pong caches, ragged chunks)
    gives, bit for bit, the GPU's causal conv of the whole sequence, and the
    final cache is its last K-1 frames (C = 256: the persistent form at the
    compiled widths)."""
    B, Tc, n = 3, 6, 9
    r = np.random.default_rng(K)
    chunks = [datagen.normal((B, Tc, C), 1.0, f"t1s/chunk/{K}/{C}/{i}", device=DEV) for i in range(n)]
    lens = [torch.as_tensor(r.integers(0, Tc + 1, B), dtype=torch.int32) for _ in range(n)]
    w = datagen.normal((K, C), 1.0 / K, f"t1s/w/{K}", device=DEV)
    b = datagen.normal((C,), 0.1, f"t1s/b/{K}", device=DEV)
    caches = [torch.zeros((B, K - 1, C), device=DEV), torch.empty((B, K - 1, C), device=DEV)]
    outs = [[] for _ in range(B)]
    for i, (x, L) in enumerate(zip(chunks, lens)):
        y, _ = lib().dwconv1d_stream_fwd(x, w, b, L.to(DEV), caches[i % 2], cache_out=caches[(i + 1) % 2])
        for bi in range(B):
            outs[bi].append(y[bi, :int(L[bi])])
    torch.cuda.synchronize()
    final = caches[n % 2]
    for bi in range(B):
        seq = torch.cat([x[bi, :int(L[bi])] for x, L in zip(chunks, lens)], dim=0)
        whole = lib().dwconv1d_fwd(seq[None].contiguous(), w, b, None, causal=True)[0]
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(outs[bi], dim=0), whole)
        tail = torch.cat([torch.zeros((K - 1, C), device=DEV), seq], dim=0)[seq.shape[0]:]
        assert torch.equal(final[bi], tail)
        assert_parity(whole, oracle.dwconv1d_fwd(seq[None], w, b, None, True)[0], TOL_F32, "whole sequence")


@pytest.mark.parametrize("Tc,C", [(12, 32), (8, 512)])
def test_empty_chunks_keep_the_cache_and_masked_frames_are_never_read(Tc, C):
    B, K = 3, 9
    x, w, b, cache, _ = make(B, Tc, C, K, lens=[0, 0, 0])
    L = torch.tensor([0, 5, Tc], dtype=torch.int32, device=DEV)
    y, c2 = check(x, w, b, cache, L, "empty and partial chunks")
    assert torch.equal(c2[0], cache[0]) and torch.all(y[0] == 0)
    xp = x.clone()
    xp[0] = float("nan")
    xp[1, 5:] = float("nan")
    y2, c3 = lib().dwconv1d_stream_fwd(xp, w, b, L, cache)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(c2, c3)


@pytest.mark.parametrize("C", [16, 256])
def test_zero_frame_chunk_copies_the_cache(C):
    B, K = 2, 5
    x, w, b, cache, _ = make(B, 1, C, K, lens=[1, 1])
    x0 = x[:, :0].contiguous()
    y, c2 = lib().dwconv1d_stream_fwd(x0, w, b, torch.zeros(B, dtype=torch.int32, device=DEV), cache)
    torch.cuda.synchronize()
    assert y.shape == (B, 0, C) and torch.equal(c2, cache)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_null_lengths_mean_full_chunks(dtype):
    """lengths = NULL: every chunk is full, the same as lengths of Tc (C = 512,
    the persistent form; C = 24, the tiled form, in fp32)."""
    for C in ((512, 24) if dtype == torch.float32 else (512,)):
        B, Tc, K = 40, 8, 9
        x, w, b, cache, _ = make(B, Tc, C, K, dtype, lens=[Tc] * B)
        full = torch.full((B,), Tc, dtype=torch.int32, device=DEV)
        y0, c0 = lib().dwconv1d_stream_fwd(x, w, b, None, cache)
        y1, c1 = lib().dwconv1d_stream_fwd(x, w, b, full, cache)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1) and torch.equal(c0, c1)
        ry, rc = oracle.dwconv1d_stream_fwd(x, w, b, None, cache)
        assert_parity(y0, ry, TOL_BF16 if dtype == torch.bfloat16 else TOL_F32, "null lengths")
        assert np.array_equal(c0.float().cpu().numpy().astype(np.float64), rc)


def test_same_cache_buffer_is_rejected():
    x, w, b, cache, L = make(2, 8, 16, 9)
    with pytest.raises(lib().DwconvError, match="different"):
        lib().dwconv1d_stream_fwd(x, w, b, L, cache, cache_out=cache)


def test_stream_workload_full():
    """1024 streams, 8-frame chunks, C = 1024, K = 9, bf16: the whole batch
    against the oracle."""
    s = datagen.conv1d_stream(device=DEV)
    L = s["lengths"].to(DEV)
    say("dwconv1d_stream full [1024,8,1024] K9 bf16")
    check(s["x"], s["w"], s["b"], s["cache"], L, "stream workload")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_unaligned_pointers_take_the_narrow_path(dtype):
    """Chunk, cache and output tensors that start one element past an aligned
    address get one-channel lanes, with the same results."""
    x, w, b, cache, L = make(3, 8, 1024, 9, dtype, lens=[8, 3, 0])

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        out = buf[1:].view(t.shape)
        out.copy_(t)
        return out

    xs, cs = shifted(x), shifted(cache)
    y = shifted(torch.zeros_like(x))
    c2 = shifted(torch.zeros_like(cache))
    say(f"dwconv1d_stream unaligned dtype={dtype}")
    lib().dwconv1d_stream_fwd(xs, w, b, L, cs, cache_out=c2, y=y)
    torch.cuda.synchronize()
    ry, rc = oracle.dwconv1d_stream_fwd(x, w, b, L, cache)
    assert_parity(y, ry, TOL_BF16 if dtype == torch.bfloat16 else TOL_F32, "unaligned")
    assert np.array_equal(c2.float().cpu().numpy().astype(np.float64), rc), "unaligned: cache differs"
