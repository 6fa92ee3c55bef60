"""GPU parity of nvfp4_quantize: codes, scales and the tensor scale must match
the oracle bit for bit (and the hand-worked golden example)."""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import announce, bf16_to_dev, to_np

pytestmark = pytest.mark.gpu


def _check(x_bits, label, rows=None, amax=None):
    announce(f"quantize {label} shape={x_bits.shape}")
    codes, scales, g = nv.quantize(bf16_to_dev(x_bits))
    torch.cuda.synchronize()
    c, s, gv = to_np(codes), to_np(scales), to_np(g)[0]
    if rows is None:
        rc, rs, rg = oracle.quantize(x_bits)
        c_cmp, s_cmp = c, s
    else:
        rc, rs, rg = oracle.quantize(x_bits[rows], amax=amax)
        c_cmp, s_cmp = c[rows], s[rows]
    assert np.float32(gv) == rg, (label, gv, rg)
    bad_s = np.argwhere(s_cmp != rs)
    assert bad_s.size == 0, (label, "scales differ at", bad_s[:5])
    bad_c = np.argwhere(c_cmp != rc)
    assert bad_c.size == 0, (label, "codes differ at", bad_c[:5], c_cmp[tuple(bad_c[0])], rc[tuple(bad_c[0])])
    return codes, scales, g


def test_hand_worked_example(golden):
    g = golden("quantize_hand_example.txt")
    rows = [[float(v) for v in g[r]] + [float(v) for v in g[r + "b"]] for r in ("row0", "row1", "row2")]
    x = workloads.to_bf16_bits(np.array(rows, np.float32))
    codes, scales, gs = nv.quantize(bf16_to_dev(x))
    c, s = to_np(codes), to_np(scales)
    assert to_np(gs)[0] == float(g["g"][0])
    for i in range(3):
        assert list(s[i]) == [int(v, 16) for v in g[f"scales{i}"]], i
        assert list(c[i]) == [int(v, 16) for v in g[f"codes{i}"]], i


def test_tiny_config():
    w = workloads.tiny()
    _check(w.x, "tiny X")
    _check(w.w, "tiny W")


@pytest.mark.parametrize("M,K,seed", [(1, 32, 1), (3, 96, 2), (300, 416, 3), (257, 1056, 4),
                                      (5, 4096, 5), (1000, 64, 6), (33, 14336, 7)])
def test_ragged_shapes(M, K, seed):
    _check(workloads.random_matrix(seed, M, K, sigma=2.0, outliers=True), f"random {M}x{K}")


def test_edge_values():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[0, :16] = 0.0                                   # all-zero block
    x[1, :16] = -0.0                                  # negative zeros
    x[2, :16] = 1e-40                                 # bf16 subnormals (tiny blocks → S = 0)
    x[2, 16:32] = np.float32(2.0 ** -126) * rng.standard_normal(16).astype(np.float32)
    x[3, :] *= 1e-6                                   # underflowing block scales
    x[4, 0] = 3.0e4                                   # tensor amax (outlier)
    _check(workloads.to_bf16_bits(x), "edge values")


def test_exact_midpoints():
    # A = 168 → g = 2^-4 exactly; the block amax 6·2^-4 gives S = 1.0 and
    # r = 16 exactly, so q lands exactly on every E2M1 midpoint
    x = np.zeros((2, 32), np.float32)
    x[0, 0] = 168.0
    mids = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                     -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 5.5], np.float32)
    x[1, :16] = mids / 16
    x[1, 16:] = -mids / 16
    codes, scales, g = _check(workloads.to_bf16_bits(x), "exact midpoints")
    assert to_np(scales)[1, 0] == 0x38 and to_np(g)[0] == 0.0625


def test_all_zero_and_domain_floor():
    z = np.zeros((8, 64), np.uint16)
    z[3, 5] = 0x8000
    _check(z, "all zero")
    x = np.zeros((4, 64), np.float32)
    x[1, 7] = 2.0 ** -100
    x[2, 9] = -(2.0 ** -101)
    _check(workloads.to_bf16_bits(x), "domain floor")


def test_qkv_activation_full():
    w = workloads.qkv()
    _check(w.x, "QKV X [4096,3072] full")


def test_qkv_weight_full():
    w = workloads.qkv()
    _check(w.w, "QKV W [9216,3072] full")


def test_long_context_sampled_rows():
    w = workloads.long_ctx()
    A = np.abs(oracle.bf16_bits_to_f32(w.x)).max()
    rows = np.r_[0:64, 16320:16448, np.random.default_rng(3).integers(0, w.M, 256), w.M - 64:w.M]
    _check(w.x, "long X [32768,3072] sampled rows", rows=np.unique(rows), amax=A)


def test_ffn_hidden_shape_sampled_rows():
    # the down projection's input has shape [8192, 14336]; the quantiser is
    # checked at that full shape on a GELU-like synthetic input
    rng = np.random.default_rng(22)
    h = rng.standard_normal((8192, 14336), dtype=np.float32) * 0.7
    h = np.where(h > 0, h, 0.05 * h).astype(np.float32)
    hb = workloads.to_bf16_bits(h)
    del h
    A = np.abs(oracle.bf16_bits_to_f32(hb)).max()
    rows = np.unique(np.r_[0:32, rng.integers(0, 8192, 200), 8160:8192])
    _check(hb, "H-shaped [8192,14336] sampled rows", rows=rows, amax=A)


@pytest.mark.parametrize("M,K,seed", [(11000, 3072, 51), (81000, 416, 52), (17000, 3072, 53)])
def test_streamed_beyond_register_capacity(M, K, seed):
    # past what 256 workgroups x 1024 threads x 8 blocks hold in registers: the
    # first two fit with 4 more blocks per thread in LDS, the third goes past
    # those 12 and streams the rest (read twice); whole-tensor bit-exactness,
    # standard and adaptive, and with the wait forced to expire
    x = workloads.random_matrix(seed, M, K, 1.0, outliers=True)
    _check(x, f"streamed {M}x{K}")
    codes, scales, g = nv.quantize(bf16_to_dev(x), adaptive46=True)
    rc, rs, rg = oracle.quantize(x, adaptive46=True)
    torch.cuda.synchronize()
    assert to_np(g)[0] == rg and np.array_equal(to_np(scales), rs) and np.array_equal(to_np(codes), rc)
    L = nv.lib()
    prev = L.nvfp4_testing_set_quantize_wait(0)
    try:
        _check(x, f"streamed {M}x{K}, wait 0")
    finally:
        L.nvfp4_testing_set_quantize_wait(prev)


def test_deterministic():
    w = workloads.qkv()
    x = bf16_to_dev(w.x)
    a = nv.quantize(x)
    b = nv.quantize(x)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_bounded_wait_fallback_gives_the_same_bytes():
    # force every workgroup of the single-launch quantiser onto the fallback
    # (its own read of the whole tensor) from the host; the bytes must not change
    L = nv.lib()
    prev = L.nvfp4_testing_set_quantize_wait(0)
    try:
        x = workloads.random_matrix(41, 1024, 3072, sigma=1.5, outliers=True)
        _check(x, "random 1024x3072, wait 0")
        codes, scales, g = nv.quantize(bf16_to_dev(x), adaptive46=True)
        rc, rs, rg = oracle.quantize(x, adaptive46=True)
        torch.cuda.synchronize()
        assert to_np(g)[0] == rg and np.array_equal(to_np(scales), rs) and np.array_equal(to_np(codes), rc)
        # two tensors in one launch (a KV append)
        rng = np.random.default_rng(42)
        k = workloads.to_bf16_bits(rng.standard_normal((100, 24, 128)).astype(np.float32))
        v = workloads.to_bf16_bits(3 * rng.standard_normal((100, 24, 128)).astype(np.float32))
        kv = nv.KVCache(100, 24, 128, max_chunks=1)
        kv.append(bf16_to_dev(k), bf16_to_dev(v))
        ref = oracle.KVCacheRef(100, 24, 128)
        ref.append(k, v)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(kv.k_codes), ref.k_codes) and np.array_equal(to_np(kv.v_scales), ref.v_scales)
        assert np.array_equal(to_np(kv.gscale)[0], np.array(ref.gscale[0], dtype=np.float32))
    finally:
        L.nvfp4_testing_set_quantize_wait(prev)
    assert L.nvfp4_testing_set_quantize_wait(prev) == prev


# ----------------------------------------------------------------------------
# The slot protocol of the single-launch quantiser on one reused workspace.
# Layout of a quantiser workspace (kernels.h): 1024 64-bit (epoch << 16 | max)
# slots from byte 0; every resident call leaves all of them with its epoch.

SLOTS_BYTES = 8192


def _into(x_dev, ws):
    M, K = x_dev.shape
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x_dev.device)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x_dev.device)
    g = torch.empty((1,), dtype=torch.float32, device=x_dev.device)
    nv.quantize_into(x_dev, codes, scales, g, ws)
    return codes, scales, g


def _assert_oracle(x_bits, out, label):
    rc, rs, rg = oracle.quantize(x_bits)
    codes, scales, g = out
    assert to_np(g)[0] == rg, (label, to_np(g)[0], rg)
    assert np.array_equal(to_np(scales), rs), label
    assert np.array_equal(to_np(codes), rc), label


@pytest.mark.parametrize("M,K", [(1024, 3072), (4096, 3072), (40, 256)])
def test_expired_wait_then_normal_wait_same_workspace(M, K):
    # A call whose waits all expire followed by a call with the normal wait on
    # smaller data, on one workspace, repeated: every call bit-exact.  (An
    # earlier protocol advanced the epoch word from workgroup 0 after an
    # expired wait, so a late workgroup could tag its slot with the next call's
    # epoch and the next call could take that stale maximum.)
    announce(f"expired wait then normal wait, {M}x{K}")
    big = workloads.random_matrix(91, M, K, sigma=4.0, outliers=True)
    small = workloads.random_matrix(92, M, K, sigma=0.25)
    ws = nv.workspace(nv.quantize_workspace_bytes(M, K))
    L = nv.lib()
    dbig, dsmall = bf16_to_dev(big), bf16_to_dev(small)
    prev = L.nvfp4_testing_set_quantize_wait(0)
    L.nvfp4_testing_set_quantize_wait(prev)
    try:
        for rep in range(6):
            L.nvfp4_testing_set_quantize_wait(0)
            o1 = _into(dbig, ws)
            L.nvfp4_testing_set_quantize_wait(prev)
            o2 = _into(dsmall, ws)
            torch.cuda.synchronize()
            _assert_oracle(big, o1, f"rep {rep} wait 0")
            _assert_oracle(small, o2, f"rep {rep} normal wait")
    finally:
        L.nvfp4_testing_set_quantize_wait(prev)


def test_kv_append_expired_wait_then_normal_wait():
    H, D, T = 24, 128, 200
    rng = np.random.default_rng(93)
    L = nv.lib()
    prev = L.nvfp4_testing_set_quantize_wait(0)
    L.nvfp4_testing_set_quantize_wait(prev)
    kv = nv.KVCache(T * 8, H, D, max_chunks=8)
    ref = oracle.KVCacheRef(T * 8, H, D)
    announce("kv append: expired wait then normal wait, one workspace")
    try:
        for rep in range(8):
            scale = 8.0 if rep % 2 == 0 else 0.125
            k = workloads.to_bf16_bits(scale * rng.standard_normal((T, H, D)).astype(np.float32))
            v = workloads.to_bf16_bits(scale * 3 * rng.standard_normal((T, H, D)).astype(np.float32))
            L.nvfp4_testing_set_quantize_wait(0 if rep % 2 == 0 else prev)
            kv.append(bf16_to_dev(k), bf16_to_dev(v))
            ref.append(k, v)
        torch.cuda.synchronize()
    finally:
        L.nvfp4_testing_set_quantize_wait(prev)
    n = kv.n_tokens
    assert np.array_equal(to_np(kv.k_codes)[:n], ref.k_codes[:n])
    assert np.array_equal(to_np(kv.v_codes)[:n], ref.v_codes[:n])
    assert np.array_equal(to_np(kv.k_scales)[:n], ref.k_scales[:n])
    assert np.array_equal(to_np(kv.v_scales)[:n], ref.v_scales[:n])
    assert np.array_equal(to_np(kv.gscale), np.array(ref.gscale, dtype=np.float32).reshape(-1, 2))


def test_stale_slots_of_earlier_calls_are_ignored():
    # A workspace in the state an earlier call leaves behind: every slot
    # tagged with that call's epoch E and holding the largest finite bf16
    # magnitude.  Calls on small data must not take any of them, and each call
    # leaves every slot with its own epoch, whatever its grid size.
    M, K = 2048, 3072
    x = workloads.random_matrix(94, M, K, sigma=0.5)
    tiny = workloads.random_matrix(95, 40, 256, sigma=0.5)
    ws = nv.workspace(nv.quantize_workspace_bytes(M, K))
    E = 0x123456789A
    slots = np.full(SLOTS_BYTES // 8, np.uint64((E << 16) | 0x7F7F), dtype=np.uint64)
    ws[:SLOTS_BYTES].copy_(torch.from_numpy(slots.view(np.uint8)))
    announce("stale slots tagged with the last completed epoch")
    for rep, xi in enumerate([x, tiny, x]):
        out = _into(bf16_to_dev(xi), ws)
        torch.cuda.synchronize()
        _assert_oracle(xi, out, f"rep {rep}")
        tags = to_np(ws[:SLOTS_BYTES]).view(np.uint64) >> np.uint64(16)
        assert np.all(tags == np.uint64(E + 1 + rep)), rep      # every slot stamped


def test_workspace_shared_by_every_kind_of_call():
    # one workspace used in turn by the single-launch path, the streamed path,
    # the two-launch 2-D path and the adaptive mode, each bit-exact
    ws = nv.workspace(nv.quantize_workspace_bytes(1, 32))
    cases = [(workloads.random_matrix(95, 3000, 3072, 1.0, True), {}),
             (workloads.random_matrix(96, 11000, 3072, 1.0, True), {}),
             (workloads.random_matrix(97, 512, 1024, 0.02), {"blocks2d": True}),
             (workloads.random_matrix(98, 3000, 3072, 0.5, True), {"adaptive46": True}),
             (workloads.random_matrix(99, 64, 256, 2.0), {})]
    for i, (x, kw) in enumerate(cases):
        announce(f"shared workspace, call {i} shape={x.shape} {kw}")
        M, K = x.shape
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
        g = torch.empty((1,), dtype=torch.float32, device="cuda")
        nv.quantize_into(bf16_to_dev(x), codes, scales, g, ws, **kw)
        torch.cuda.synchronize()
        rc, rs, rg = oracle.quantize(x, **kw)
        assert to_np(g)[0] == rg and np.array_equal(to_np(scales), rs) and np.array_equal(to_np(codes), rc), i


def test_one_buffer_shared_by_every_entry_point():
    # Every workspace starts with the same head (the scratch of two quantised
    # tensors) and keeps its other buffers after it, so one zeroed buffer can
    # serve linear layers of different sizes, quantisation, KV appends, the
    # QKV append, the Hadamard-transformed quantiser and attention in turn.
    # Each result equals the same call on a workspace of its own (or the
    # oracle), and afterwards each of the two slot regions carries one tag:
    # no call has written data where another keeps its slots.
    H, D, T, Dm = 24, 128, 880, 3072
    rng_w = [workloads.random_matrix(200 + i, n, k, sigma=0.02) for i, (n, k) in
             enumerate([(1024, 3072), (512, 1024), (3 * H * D, Dm)])]
    wq = [nv.quantize(bf16_to_dev(w)) for w in rng_w]
    x1 = bf16_to_dev(workloads.random_matrix(210, 512, 3072, sigma=1.0, outliers=True))
    x2 = bf16_to_dev(workloads.random_matrix(211, 2048, 1024, sigma=2.0, outliers=True))
    xq = workloads.random_matrix(212, 3000, 3072, sigma=0.5, outliers=True)
    xr = workloads.random_matrix(213, 512, 3072, sigma=1.0)
    xf = bf16_to_dev(workloads.random_matrix(214, T, Dm, sigma=1.0, outliers=True))
    kvs = [workloads.random_matrix(215 + i, T, H * D, sigma=1.0 + i) for i in range(4)]
    q = bf16_to_dev(workloads.random_matrix(220, 256, H * D, sigma=1.0))
    shared = nv.KVCache(4 * T, H, D, max_chunks=8)
    fresh = nv.KVCache(4 * T, H, D, max_chunks=8)
    need = max(nv.linear_workspace_bytes(512, 3072), nv.linear_workspace_bytes(2048, 1024),
               nv.quantize_workspace_bytes(3000, 3072), shared.workspace_bytes(T),
               shared.qkv_workspace_bytes(T, Dm), nv.quantize_rht_workspace_bytes(512, 3072),
               nv.attention_workspace_bytes(256, H, 2 * T), nv.attention_workspace_bytes(256, H, 3 * T))
    ws = nv.workspace(need)
    announce(f"one {need}-byte workspace for every entry point")
    for rep in range(2):
        for x, w in ((x1, wq[0]), (x2, wq[1])):
            got = nv.linear(x, *w, ws=ws)
            assert torch.equal(got, nv.linear(x, *w)), ("linear", rep, tuple(x.shape))
        codes = torch.empty((3000, 1536), dtype=torch.uint8, device="cuda")
        scales = torch.empty((3000, 192), dtype=torch.uint8, device="cuda")
        g = torch.empty((1,), dtype=torch.float32, device="cuda")
        nv.quantize_into(bf16_to_dev(xq), codes, scales, g, ws)
        _assert_oracle(xq, (codes, scales, g), f"quantize rep {rep}")
        k, v = (bf16_to_dev(kvs[2 * rep]), bf16_to_dev(kvs[2 * rep + 1]))
        shared.append(k, v, ws=ws)
        fresh.append(k, v)
        if rep == 0:
            shared.qkv_append(xf, *wq[2], ws=ws)
            fresh.qkv_append(xf, *wq[2])
        rc, rs, rg = nv.quantize_rht(bf16_to_dev(xr), 0xA5C3, ws=ws)
        oc, os_, og = oracle.quantize_rht(xr, 0xA5C3)
        assert np.array_equal(to_np(rc), oc) and np.array_equal(to_np(rs), os_) and to_np(rg)[0] == og
        n = shared.n_tokens
        o_shared = shared.attention(q, [(0, n)], ws=ws)
        assert torch.equal(o_shared, fresh.attention(q, [(0, n)])), ("attention", rep)
    torch.cuda.synchronize()
    n = shared.n_tokens
    for a, b in ((shared.k_codes, fresh.k_codes), (shared.v_codes, fresh.v_codes),
                 (shared.k_scales, fresh.k_scales), (shared.v_scales, fresh.v_scales)):
        assert torch.equal(a[:n], b[:n])
    assert torch.equal(shared.gscale[:shared.n_chunks], fresh.gscale[:fresh.n_chunks])
    for r, off in enumerate((0, 12288)):
        tags = to_np(ws[off:off + SLOTS_BYTES]).view(np.uint64) >> np.uint64(16)
        assert len(set(tags.tolist())) == 1, ("slot region", r)
