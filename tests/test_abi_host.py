"""C-ABI library on the host: it loads, exports every declared symbol, and
rejects bad arguments before anything reaches the device (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsv.h")


@pytest.fixture(scope="module")
def hsv():
    from long_context_tree_verify_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from long_context_tree_verify_amd import build_lib
        build_lib.build()
    import long_context_tree_verify_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hsv_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(hsv):
    names = declared_functions()
    assert len(names) >= 8
    assert set(names) == set(hsv.EXPORTS)
    lib = ctypes.CDLL(hsv._lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(hsv):
    for code in range(7):
        s = hsv.hsv_status_string(code)
        assert s.startswith("HSV_")
    assert "unknown" in hsv.hsv_status_string(99)
    assert hsv.hsv_version() == 1


def _desc(hsv, **kw):
    base = dict(batch=1, n_draft=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
                kv_capacity=32832, max_ctx=32768)
    base.update(kw)
    return hsv.make_desc(**base)


def _ws(hsv, d):
    n = ctypes.c_size_t(0)
    code = hsv.lib.hsv_verify_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
    return code, n.value


def test_workspace_size_valid_and_monotone(hsv):
    code, n = _ws(hsv, _desc(hsv))
    assert code == hsv.HSV_OK and n > 0
    prev = 0
    for splits in (1, 2, 7, 32, 256):
        code, m = _ws(hsv, _desc(hsv, num_splits=splits))
        assert code == hsv.HSV_OK and m > prev
        prev = m
    # the tree part alone needs one part's worth
    code, t = _ws(hsv, _desc(hsv, flags=hsv.HSV_FLAG_NO_PREFIX))
    assert code == hsv.HSV_OK and t < n


def test_empty_key_set_plan_has_no_partials(hsv):
    """No prefix keys and no tree part: the plan holds no partial rows, so the
    workspace is the error word alone (256 bytes) and the merge kernel must
    not read partials (it writes o = 0, lse = -inf instead)."""
    for kw in (dict(), dict(n_draft=8), dict(n_q_heads=16, n_draft=32, head_dim=64),
               dict(n_q_heads=1, n_kv_heads=1, n_draft=8, head_dim=64, in_dtype=hsv.HSV_F32)):
        code, n = _ws(hsv, _desc(hsv, max_ctx=0, flags=hsv.HSV_FLAG_NO_TREE, **kw))
        assert code == hsv.HSV_OK and n == 256, kw


@pytest.mark.parametrize("kw,code", [
    (dict(n_draft=0), 2), (dict(n_draft=257), 2), (dict(batch=0), 2),
    (dict(n_draft=65, head_dim=64, max_ctx=32000), 0),
    (dict(n_draft=65, n_q_heads=8, max_ctx=32000), 0), (dict(n_draft=256, max_ctx=32000), 0),
    (dict(n_draft=200, n_q_heads=8, head_dim=64, max_ctx=32000, in_dtype=0), 0),
    (dict(n_q_heads=30), 2), (dict(n_kv_heads=0), 2), (dict(head_dim=96), 3),
    (dict(max_ctx=32769), 2), (dict(max_ctx=-1), 2), (dict(num_splits=257), 2),
    (dict(num_splits=-1), 2), (dict(in_dtype=7), 3), (dict(out_dtype=2), 3),
    (dict(scale=-1.0), 2), (dict(scale=float("nan")), 2), (dict(flags=64), 3),
    (dict(flags=6), 2), (dict(n_sel=5000, max_ctx=4000), 2), (dict(flags=128), 3),
    (dict(flags=32), 0),
])
def test_workspace_rejects_bad_descriptors(hsv, kw, code):
    got, _ = _ws(hsv, _desc(hsv, **kw))
    assert got == code


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: the calls below fail first


def _call_dense(hsv, d, q=FAKE, k=FAKE, v=FAKE, ctx=FAKE, parent=FAKE, anc=None, o=FAKE,
                lse=FAKE, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = _ws(hsv, d)[1]
    return hsv.lib.hsv_verify_attn(ctypes.byref(d), q, k, v, ctx, parent, anc, o, lse, ws,
                                   ctypes.c_size_t(ws_bytes), None)


def test_verify_rejects_null_and_workspace_errors(hsv):
    d = _desc(hsv)
    assert _call_dense(hsv, d, q=None) == hsv.HSV_ERR_NULL
    assert _call_dense(hsv, d, lse=None) == hsv.HSV_ERR_NULL
    assert _call_dense(hsv, d, parent=None) == hsv.HSV_ERR_NULL           # neither
    assert _call_dense(hsv, d, anc=FAKE) == hsv.HSV_ERR_NULL              # both
    assert _call_dense(hsv, d, ws=None) == hsv.HSV_ERR_WORKSPACE
    assert _call_dense(hsv, d, ws_bytes=100) == hsv.HSV_ERR_WORKSPACE
    assert _call_dense(hsv, d, ws=ctypes.c_void_p(0x10010)) == hsv.HSV_ERR_WORKSPACE
    assert _call_dense(hsv, d, k=ctypes.c_void_p(0x10002)) == hsv.HSV_ERR_SHAPE
    assert hsv.lib.hsv_verify_attn(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                   ctypes.c_size_t(1 << 20), None) == hsv.HSV_ERR_NULL
    bad = _desc(hsv, n_draft=257)
    assert _call_dense(hsv, bad, ws_bytes=1 << 30) == hsv.HSV_ERR_SHAPE
    # a dense call must not carry n_sel; the tree may be left out without parents
    assert _call_dense(hsv, _desc(hsv, n_sel=10), ws_bytes=1 << 30) == hsv.HSV_ERR_SHAPE


def test_sparse_rejects_missing_indices(hsv):
    d = _desc(hsv, n_sel=4096)
    n = _ws(hsv, d)[1]
    code = hsv.lib.hsv_verify_attn_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          None, FAKE, FAKE, FAKE, ctypes.c_size_t(n), None)
    assert code == hsv.HSV_ERR_NULL
    d0 = _desc(hsv, n_sel=0)
    code = hsv.lib.hsv_verify_attn_sparse(ctypes.byref(d0), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          FAKE, FAKE, FAKE, FAKE, ctypes.c_size_t(1 << 30), None)
    assert code == hsv.HSV_ERR_SHAPE


def test_small_entry_points_reject_bad_arguments(hsv):
    lib = hsv.lib
    assert lib.hsv_tree_ancestor_mask(None, FAKE, 1, 8, None) == hsv.HSV_ERR_NULL
    assert lib.hsv_tree_ancestor_mask(FAKE, FAKE, 1, 257, None) == hsv.HSV_ERR_SHAPE
    assert lib.hsv_tree_ancestor_mask(FAKE, FAKE, 0, 8, None) == hsv.HSV_ERR_SHAPE
    assert lib.hsv_gather_kv(FAKE, FAKE, None, FAKE, FAKE, 1, 1, 10, 128, 4, 1,
                             None) == hsv.HSV_ERR_NULL
    assert lib.hsv_gather_kv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 10, 80, 4, 1,
                             None) == hsv.HSV_ERR_UNSUPPORTED
    assert lib.hsv_gather_kv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 10, 128, 0, 1,
                             None) == hsv.HSV_ERR_SHAPE
    assert lib.hsv_lse_merge(FAKE, FAKE, 0, 10, 128, FAKE, FAKE, 0, None) == hsv.HSV_ERR_SHAPE
    assert lib.hsv_lse_merge(FAKE, None, 2, 10, 128, FAKE, FAKE, 0, None) == hsv.HSV_ERR_NULL
    assert lib.hsv_lse_merge(FAKE, FAKE, 2, 10, 32, FAKE, FAKE, 0, None) == \
        hsv.HSV_ERR_UNSUPPORTED


def test_product_package_does_not_reach_the_oracle():
    pkg = os.path.join(ROOT, "long_context_tree_verify_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h", ".hpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "liboracle" not in text, f
                assert "from oracle" not in text, f


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=64), 0), (dict(block_size=256), 0), (dict(block_size=16), 2),
    (dict(block_size=96), 2), (dict(block_size=128, kv_capacity=32832), 2),
    (dict(block_size=64, n_sel=100), 3),                         # sparse, 256 rows: MFMA
    (dict(block_size=64, n_sel=100, n_draft=8), 0),              # sparse, 32 rows
    (dict(block_size=64, n_sel=100, n_draft=8, max_ctx=393208, kv_capacity=393216), 0),
    (dict(block_size=64, n_sel=100, n_draft=8, max_ctx=393216, kv_capacity=393280), 3),
    (dict(block_size=64, n_sel=100, n_draft=8, flags=2), 3),     # sparse, no prefix
    (dict(block_size=64, flags=2), 3),                           # no prefix
    (dict(block_size=64, n_draft=16, n_q_heads=32), 3),          # 64 rows: MFMA kernel
    (dict(block_size=64, head_dim=64), 3),                       # D 64
    (dict(block_size=64, max_ctx=600000, kv_capacity=600064), 3),  # > 256 splits of 2048 keys
    # one (sequence, KV head) on the small-group kernel: the split target for
    # all of the CUs' workgroups exceeds the split limit and is clamped to it
    (dict(block_size=1024, batch=1, n_q_heads=1, n_kv_heads=1, n_draft=5, max_ctx=100,
          kv_capacity=1024), 0),
])
def test_paged_descriptors(hsv, kw, code):
    if kw.get("block_size") and "kv_capacity" not in kw:
        kw["kv_capacity"] = 32832 if 32832 % kw["block_size"] == 0 else 32768 + kw["block_size"]
    got, n = _ws(hsv, _desc(hsv, **kw))
    assert got == code
    if code == 0:
        assert n > 0


def test_paged_call_argument_errors(hsv):
    d = _desc(hsv, block_size=64)
    n = _ws(hsv, d)[1]

    def call(desc, table=FAKE, n_pool=10):
        return hsv.lib.hsv_verify_attn_paged(ctypes.byref(desc), FAKE, FAKE, FAKE, table, n_pool,
                                             FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                             ctypes.c_size_t(n), None)

    assert call(d, table=None) == hsv.HSV_ERR_NULL
    assert call(d, n_pool=0) == hsv.HSV_ERR_SHAPE

    ds = _desc(hsv, block_size=64, n_sel=100, n_draft=8)
    ns = _ws(hsv, ds)[1]

    def call_sparse(desc, table=FAKE, kv_idx=FAKE, n_pool=10):
        return hsv.lib.hsv_verify_attn_sparse_paged(
            ctypes.byref(desc), FAKE, FAKE, FAKE, table, n_pool, FAKE, FAKE, None, kv_idx,
            FAKE, FAKE, FAKE, ctypes.c_size_t(ns), None)

    assert call_sparse(ds, table=None) == hsv.HSV_ERR_NULL
    assert call_sparse(ds, kv_idx=None) == hsv.HSV_ERR_NULL
    assert call_sparse(ds, n_pool=0) == hsv.HSV_ERR_SHAPE
    assert call_sparse(_desc(hsv, n_sel=100, n_draft=8)) == hsv.HSV_ERR_SHAPE  # no block size
    assert call_sparse(_desc(hsv, block_size=64, n_draft=8)) == hsv.HSV_ERR_SHAPE  # n_sel 0
    assert call(_desc(hsv)) == hsv.HSV_ERR_SHAPE                 # no block size
    # a contiguous call must not carry a block size
    assert _call_dense(hsv, d, ws_bytes=n) == hsv.HSV_ERR_SHAPE
