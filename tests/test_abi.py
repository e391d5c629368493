"""The C-ABI library on the host: it loads, exports what include/mcs.h declares,
and rejects bad arguments before touching the GPU (every call below fails
validation, so nothing is enqueued and no GPU is needed)."""
import ctypes

import pytest

import sparse_attention_diffusion_attn_amd as mcs

P = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10008        # misaligned


def d(batch=1, heads=2, n_valid=1000, n_pad=1024, head_dim=128, group_size=128):
    return mcs.make_dims(batch, heads, n_valid, n_pad, head_dim, group_size)


def err():
    return mcs.lib().mcs_last_error().decode()


def test_library_exports_every_header_symbol():
    lib = mcs.lib()
    names = mcs.header_functions()
    assert set(names) >= {"mcs_group", "mcs_anchor_select", "mcs_residual", "mcs_sparse_attn",
                          "mcs_dense_attn", "mcs_group_workspace_bytes",
                          "mcs_anchor_select_workspace_bytes", "mcs_anchor_select_min_workspace_bytes",
                          "mcs_status_string", "mcs_last_error", "mcs_abi_version"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mcs_abi_version() == 2
    assert lib.mcs_status_string(3) == b"MCS_ERR_WORKSPACE"
    assert lib.mcs_status_string(99) == b"MCS_ERR_UNKNOWN"


def test_workspace_sizes():
    lib = mcs.lib()
    dm = d()
    G, bh, D = 8, 2, 128
    want = 0
    # partials, mu, v, projections, second perm, then the covariance path:
    # chunk partials of the formed nodes at the depth that needs most (G = 8,
    # 3 depths: the root in 1 chunk, 1 left child of 4 groups, 2 left
    # children of 2 groups: 2 entries) and two buffers of kept entries
    # (2^(3-2) = 2 slots); an entry is 36 upper 16x16 fp64 tiles + 128 row sums
    e = (36 * 256 + 128) * 8
    for nbytes in (bh * G * D * 8,) * 3 + (bh * 1024 * 8, bh * 1024 * 4, bh * 2 * e, bh * 2 * e, bh * 2 * e):
        want = (want + nbytes + 255) // 256 * 256
    assert lib.mcs_group_workspace_bytes(ctypes.byref(dm)) == want
    per_head = (G * 1000 * 4 + 255) // 256 * 256 + (G * 1024 * 4 + 255) // 256 * 256
    assert lib.mcs_anchor_select_min_workspace_bytes(ctypes.byref(dm), 250) == per_head
    assert lib.mcs_anchor_select_workspace_bytes(ctypes.byref(dm), 250) == 2 * per_head
    assert lib.mcs_anchor_select_workspace_bytes(ctypes.byref(dm), 0) == 0
    assert lib.mcs_group_workspace_bytes(ctypes.byref(d(head_dim=80))) == 0
    assert lib.mcs_group_workspace_bytes(ctypes.byref(d(head_dim=96))) > 0


@pytest.mark.parametrize("kw,code,msg", [
    (dict(head_dim=80), mcs.MCS_ERR_UNSUPPORTED, "head_dim"),
    (dict(head_dim=256), mcs.MCS_ERR_UNSUPPORTED, "head_dim"),
    (dict(group_size=32), mcs.MCS_ERR_UNSUPPORTED, "group_size"),
    (dict(n_pad=1000, n_valid=900), mcs.MCS_ERR_INVALID_ARG, "multiple"),
    (dict(n_valid=0), mcs.MCS_ERR_INVALID_ARG, "n_valid"),
    (dict(n_valid=2000), mcs.MCS_ERR_INVALID_ARG, "n_valid"),
    (dict(batch=0), mcs.MCS_ERR_INVALID_ARG, "batch"),
    (dict(n_pad=1 << 25, n_valid=10), mcs.MCS_ERR_UNSUPPORTED, "n_pad"),
])
def test_bad_dims_rejected_by_every_call(kw, code, msg):
    lib = mcs.lib()
    dm = d(**kw)
    b = ctypes.byref(dm)
    calls = [
        lambda: lib.mcs_group(b, P, 20, -1, P, P, 1 << 30, None),
        lambda: lib.mcs_anchor_select(b, P, P, P, P, 5, 0.1, P, P, P, P, 1 << 30, None),
        lambda: lib.mcs_residual(b, P, P, P, P, P, 5, 0.1, P, P, None),
        lambda: lib.mcs_sparse_attn(b, P, P, P, P, P, 5, 0.1, None, P + 256, None),
        lambda: lib.mcs_dense_attn(b, P, P, P, 0.1, P + 256, None, None),
    ]
    for c in calls:
        assert c() == code
        assert msg in err()


def test_argument_checks():
    lib = mcs.lib()
    b = ctypes.byref(d())
    # null and misaligned pointers
    assert lib.mcs_sparse_attn(b, None, P, P, P, P, 5, 0.1, None, P + 256, None) == mcs.MCS_ERR_INVALID_ARG
    assert "q is NULL" in err()
    assert lib.mcs_sparse_attn(b, P, MIS, P, P, P, 5, 0.1, None, P + 256, None) == mcs.MCS_ERR_INVALID_ARG
    assert "k is not 16-byte aligned" in err()
    assert lib.mcs_dense_attn(b, P, P, P, 0.1, None, None, None) == mcs.MCS_ERR_INVALID_ARG
    assert lib.mcs_residual(b, P, P, P, P, P, 5, 0.1, None, P, None) == mcs.MCS_ERR_INVALID_ARG
    # topk range
    for k in (0, 1001, -3):
        assert lib.mcs_sparse_attn(b, P, P, P, P, P, k, 0.1, None, P + 256, None) == mcs.MCS_ERR_INVALID_ARG
        assert "topk" in err()
        assert lib.mcs_anchor_select(b, P, P, P, P, k, 0.1, P, P, P, P, 1 << 30, None) == mcs.MCS_ERR_INVALID_ARG
    # scale
    for sc in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.mcs_dense_attn(b, P, P, P, sc, P + 256, None, None) == mcs.MCS_ERR_INVALID_ARG
        assert "scale" in err()
    # aliasing output
    assert lib.mcs_sparse_attn(b, P, P + 16, P + 32, P, P, 5, 0.1, None, P, None) == mcs.MCS_ERR_INVALID_ARG
    assert "alias" in err()
    # grouping arguments
    assert lib.mcs_group(b, P, -1, -1, P, P, 1 << 30, None) == mcs.MCS_ERR_INVALID_ARG
    assert lib.mcs_group(b, P, 20, 4, P, P, 1 << 30, None) == mcs.MCS_ERR_INVALID_ARG  # L = 3
    assert "max_levels" in err()


def test_workspace_checks():
    lib = mcs.lib()
    dm = d()
    b = ctypes.byref(dm)
    need = lib.mcs_group_workspace_bytes(b)
    assert lib.mcs_group(b, P, 20, -1, P, P, need - 1, None) == mcs.MCS_ERR_WORKSPACE
    assert lib.mcs_group(b, P, 20, -1, P, None, need, None) == mcs.MCS_ERR_WORKSPACE
    assert lib.mcs_group(b, P, 20, -1, P, P + 16, need, None) == mcs.MCS_ERR_WORKSPACE
    assert "256-byte" in err()
    mn = lib.mcs_anchor_select_min_workspace_bytes(b, 5)
    assert lib.mcs_anchor_select(b, P, P, P, P, 5, 0.1, P + 256, P, P, P, mn - 1, None) == mcs.MCS_ERR_WORKSPACE


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mcs.dense_attn(q, q, q, 128, 64)


def test_block_select_checks():
    lib = mcs.lib()
    dm = d()                       # n_valid 1000, C 128, 2 heads
    b = ctypes.byref(dm)
    ws = lib.mcs_block_select_workspace_bytes(b, mcs.BLOCK_EXACT, 64, 4)
    mn = lib.mcs_block_select_min_workspace_bytes(b, mcs.BLOCK_EXACT, 64, 4)
    G, NB = 8, 16
    per_head = sum((x + 255) // 256 * 256 for x in (G * 1000 * 4, G * NB * 4, G * 4 * 4))
    assert mn == per_head and ws == 2 * per_head
    per_head_mp = sum((x + 255) // 256 * 256 for x in (NB * 128 * 8, G * NB * 4, G * 4 * 4))
    assert lib.mcs_block_select_min_workspace_bytes(b, mcs.BLOCK_MEANPOOL, 64, 4) == per_head_mp
    assert lib.mcs_block_select_workspace_bytes(b, 7, 64, 4) == 0
    call = lambda mode, blk, nb, lse=P, wsb=1 << 30: lib.mcs_block_select(  # noqa: E731
        b, P, P, P, lse, mode, blk, nb, 0.1, P, P, P, wsb, None)
    assert call(2, 64, 4) == mcs.MCS_ERR_INVALID_ARG and "mode" in err()
    assert call(mcs.BLOCK_EXACT, 0, 4) == mcs.MCS_ERR_INVALID_ARG and "block" in err()
    assert call(mcs.BLOCK_EXACT, 64, 17) == mcs.MCS_ERR_INVALID_ARG and "nblocks" in err()
    assert call(mcs.BLOCK_EXACT, 1, 1001) == mcs.MCS_ERR_INVALID_ARG and "nblocks" in err()
    assert call(mcs.BLOCK_EXACT, 64, 4, lse=None) == mcs.MCS_ERR_INVALID_ARG and "lse" in err()
    assert call(mcs.BLOCK_EXACT, 64, 4, wsb=mn - 1) == mcs.MCS_ERR_WORKSPACE


def test_counts_calls_checks():
    lib = mcs.lib()
    b = ctypes.byref(d())
    assert lib.mcs_sparse_attn_counts(b, P, P, P, P, P, 0, P, 0.1, None, P + 256, None) == mcs.MCS_ERR_INVALID_ARG
    assert "kv_stride" in err()
    assert lib.mcs_sparse_attn_counts(b, P, P, P, P, P, 8, None, 0.1, None, P + 256, None) == mcs.MCS_ERR_INVALID_ARG
    assert "kv_count" in err()
    assert lib.mcs_residual_counts(b, P, P, P, P, P, 8, P, 0.1, None, P + 256, None) == mcs.MCS_ERR_INVALID_ARG
    assert "o_full" in err()
    assert lib.mcs_sparse_attn_counts(b, P, P, P, P, P, 8, P, 0.1, None, P, None) == mcs.MCS_ERR_INVALID_ARG
    assert "alias" in err()
    # R is written while the kernel reads K/V rows of other tokens: it may not
    # alias q, k or v
    q, k, v = P, P + 0x100000, P + 0x200000
    for r in (q, k, v):
        assert lib.mcs_residual_counts(b, q, k, v, P, P, 8, P, 0.1, P + 0x300000, r, None) == \
            mcs.MCS_ERR_INVALID_ARG
        assert "alias" in err()


def _layout(fn, dm):
    lay = mcs.Layout()
    fn(ctypes.byref(dm), ctypes.byref(lay))
    return lay


def test_layout_helpers():
    lib = mcs.lib()
    dm = d(batch=2, heads=3, n_pad=1024, head_dim=64)
    a = _layout(lib.mcs_layout_bhnd, dm)
    b = _layout(lib.mcs_layout_bnhd, dm)
    for t in (a.q, a.k, a.v, a.o):
        assert (t.batch, t.head, t.token) == (3 * 1024 * 64, 1024 * 64, 64)
    for t in (b.q, b.k, b.v, b.o):
        assert (t.batch, t.head, t.token) == (1024 * 3 * 64, 64, 3 * 64)


def test_strided_layout_checks():
    """Every bad layout is refused before anything is enqueued."""
    lib = mcs.lib()
    dm = d(batch=2, heads=3)
    b = ctypes.byref(dm)

    def calls(lay):
        lp = ctypes.byref(lay)
        return [
            lambda: lib.mcs_group_strided(b, lp, P, 20, -1, P, P, 1 << 30, None),
            lambda: lib.mcs_anchor_select_strided(b, lp, P, P, P, P, 5, 0.1, P + 256, P, P, P,
                                                  1 << 30, None),
            lambda: lib.mcs_residual_strided(b, lp, P, P, P, P, P, 5, 0.1, P, P + 256, None),
            lambda: lib.mcs_sparse_attn_strided(b, lp, P, P, P, P, P, 5, 0.1, None, P + 256, None),
            lambda: lib.mcs_dense_attn_strided(b, lp, P, P, P, 0.1, P + 256, None, None),
        ]

    def bad(mutate, code, msg, only=None):
        lay = _layout(lib.mcs_layout_bnhd, dm)
        mutate(lay)
        cs = calls(lay)
        for c in (cs if only is None else [cs[i] for i in only]):
            assert c() == code, msg
            assert msg in err()

    def set_(name, field, value):
        return lambda lay: setattr(getattr(lay, name), field, value)

    bad(set_("q", "token", 3 * 128 + 4), mcs.MCS_ERR_INVALID_ARG, "multiple of 8")
    bad(set_("q", "head", -128), mcs.MCS_ERR_INVALID_ARG, "outside")
    bad(set_("k", "batch", 1 << 41), mcs.MCS_ERR_INVALID_ARG, "outside", only=[1, 2, 3, 4])
    bad(set_("k", "token", 1 << 23), mcs.MCS_ERR_UNSUPPORTED, "token stride", only=[1, 2, 3, 4])
    # one head's rows must fit a 32-bit byte offset: 1023 rows of 2^22 elements
    bad(set_("v", "token", 1 << 22), mcs.MCS_ERR_UNSUPPORTED, "4 GiB", only=[1, 2, 3, 4])
    bad(set_("v", "token", 3 * 128 * 2), mcs.MCS_ERR_UNSUPPORTED, "share the token stride",
        only=[1, 2, 3, 4])
    # overlapping output rows (token stride below the row length, or heads on top of each other)
    bad(set_("o", "token", 64), mcs.MCS_ERR_INVALID_ARG, "overlap", only=[1, 2, 3, 4])
    bad(set_("o", "head", 0), mcs.MCS_ERR_INVALID_ARG, "overlap", only=[1, 2, 3, 4])
    bad(set_("o", "batch", 1024 * 3 * 128 - 8), mcs.MCS_ERR_INVALID_ARG, "overlap",
        only=[1, 2, 3, 4])


def test_strided_extent_one_strides_ignored_and_alias_rules():
    """A stride of a dimension of extent 1 is not checked; R may overwrite
    O_full only when O_full is contiguous."""
    lib = mcs.lib()
    dm = d(batch=1, heads=2)
    b = ctypes.byref(dm)
    lay = _layout(lib.mcs_layout_bnhd, dm)
    lay.q.batch = 3           # extent 1: ignored ...
    lay.q.token = 3           # ... but this one is not
    assert lib.mcs_dense_attn_strided(b, ctypes.byref(lay), P, P, P, 0.1, P + 256, None,
                                      None) == mcs.MCS_ERR_INVALID_ARG
    assert "q token stride" in err()
    lay = _layout(lib.mcs_layout_bnhd, dm)
    assert lib.mcs_residual_strided(b, ctypes.byref(lay), P, P, P, P, P, 5, 0.1, P + 256,
                                    P + 256, None) == mcs.MCS_ERR_INVALID_ARG
    assert "o_full is contiguous" in err()
    assert lib.mcs_residual_strided(b, ctypes.byref(lay), P, P, P, P, P, 5, 0.1, P + 256,
                                    P, None) == mcs.MCS_ERR_INVALID_ARG
    assert "alias" in err()
    assert lib.mcs_anchor_select_strided(b, ctypes.byref(lay), P, P, P, P, 5, 0.1, P, P, P, P,
                                         1 << 30, None) == mcs.MCS_ERR_INVALID_ARG
    assert "alias" in err()
    assert lib.mcs_dense_attn_strided(b, ctypes.byref(lay), P, P, P, 0.1, P, None,
                                      None) == mcs.MCS_ERR_INVALID_ARG
    assert "alias" in err()


def test_kmeans_checks():
    lib = mcs.lib()
    dm = d()                                  # 2 heads, n_pad 1024, d 128, C 128: 8 groups
    b = ctypes.byref(dm)
    G, bh, tiles = 8, 2, 1
    want = 0
    for nbytes in (bh * 1024 * 4, bh * 1024 * 4, bh * G * 128 * 2, bh * G * 4, bh * tiles * G * 4):
        want = (want + nbytes + 255) // 256 * 256
    need = lib.mcs_group_kmeans_workspace_bytes(b)
    assert need == want
    big = mcs.make_dims(1, 1, 8193 * 64, 8193 * 64, 64, 64)
    assert lib.mcs_group_kmeans_workspace_bytes(ctypes.byref(big)) == 0
    assert lib.mcs_group_kmeans(ctypes.byref(big), P, 3, P, None, P, 1 << 30, None) == mcs.MCS_ERR_UNSUPPORTED
    assert "8192" in err()
    assert lib.mcs_group_kmeans(b, P, -1, P, None, P, need, None) == mcs.MCS_ERR_INVALID_ARG
    assert "iters" in err()
    assert lib.mcs_group_kmeans(b, P, 1001, P, None, P, need, None) == mcs.MCS_ERR_INVALID_ARG
    assert lib.mcs_group_kmeans(b, P, 3, None, None, P, need, None) == mcs.MCS_ERR_INVALID_ARG
    assert lib.mcs_group_kmeans(b, P, 3, P, MIS, P, need, None) == mcs.MCS_ERR_INVALID_ARG
    assert lib.mcs_group_kmeans(b, P, 3, P, None, P, need - 1, None) == mcs.MCS_ERR_WORKSPACE
    assert lib.mcs_group_kmeans(b, P, 3, P, None, P + 16, need, None) == mcs.MCS_ERR_WORKSPACE


def test_noalloc_validation_before_any_gpu_work():
    """mcs_anchor_select_noalloc rejects, on the host, shapes whose single head
    needs more than the fixed scratch, and bad shapes as mcs_anchor_select does."""
    lib = mcs.lib()
    hy = d(heads=1, n_valid=118800, n_pad=118912)
    need = lib.mcs_anchor_select_min_workspace_bytes(ctypes.byref(hy), 29700)
    assert need > mcs.NOALLOC_SCRATCH_BYTES
    assert lib.mcs_anchor_select_noalloc(ctypes.byref(hy), P, P, P, P, 29700, 0.1, P, P, P, None) == \
        mcs.MCS_ERR_UNSUPPORTED
    assert "scratch" in err()
    assert lib.mcs_anchor_select_noalloc(ctypes.byref(d(head_dim=80)), P, P, P, P, 10, 0.1, P, P, P, None) == \
        mcs.MCS_ERR_UNSUPPORTED
    assert "head_dim" in err()
    assert lib.mcs_anchor_select_noalloc(ctypes.byref(d()), P, P, P, P, 0, 0.1, P, P, P, None) == \
        mcs.MCS_ERR_INVALID_ARG
    assert "topk" in err()


def test_head_dim_96_scope():
    """d = 96 runs through the five calls of the method; the k-means
    comparator and the block-selection variants stay at d = 64 and 128."""
    lib = mcs.lib()
    d96 = d(head_dim=96)
    assert lib.mcs_anchor_select_workspace_bytes(ctypes.byref(d96), 250) > 0
    assert lib.mcs_group_kmeans_workspace_bytes(ctypes.byref(d96)) == 0
    assert lib.mcs_group_kmeans(ctypes.byref(d96), P, 3, P, None, P, 1 << 30, None) == mcs.MCS_ERR_UNSUPPORTED
    assert "k-means" in err()
    assert lib.mcs_block_select_workspace_bytes(ctypes.byref(d96), mcs.BLOCK_EXACT, 64, 4) == 0
    assert lib.mcs_block_select(ctypes.byref(d96), P, P, P, P, mcs.BLOCK_EXACT, 64, 4, 0.1, P, P, P,
                                1 << 30, None) == mcs.MCS_ERR_UNSUPPORTED
    assert "block selection" in err()
