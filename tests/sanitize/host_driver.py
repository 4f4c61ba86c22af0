"""Drives the host side of libhsv.so (descriptor checks, planning, workspace
sizing, argument validation) for a build whose host code runs under
AddressSanitizer and UndefinedBehaviorSanitizer.

usage: python host_driver.py LIBRARY

Only calls that must fail before any device work are made, so no GPU is
needed: seeded random descriptors (valid and malformed, sizes up to the
int32 limits) through the workspace-size queries, and every entry point with
missing pointers, malformed shapes or short workspaces.  The binding's
ctypes declarations are loaded from its file, without the package (and
without torch).  Exit status 0 when every call returned an hsv_status and
every rejected call returned the status its contract names.
"""

import ctypes
import importlib.util
import os
import random
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIBFILE = os.path.join(HERE, "..", "..", "long_context_tree_verify_amd", "_lib.py")


def load_binding(path):
    spec = importlib.util.spec_from_file_location("hsv_lib_decls", LIBFILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.LIB_PATH = path
    return mod, mod.load()


def main(argv):
    m, lib = load_binding(argv[1])
    rng = random.Random(20261203)
    failures = []
    sz = ctypes.c_size_t
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails first

    def desc(**kw):
        d = m.HsvVerifyDesc()
        base = dict(batch=1, n_draft=64, n_q_heads=32, n_kv_heads=8, head_dim=128,
                    kv_capacity=32832, max_ctx=32768, n_sel=0, in_dtype=m.HSV_BF16,
                    out_dtype=m.HSV_BF16, scale=0.0, num_splits=0, flags=0, block_size=0)
        base.update(kw)
        for k, v in base.items():
            setattr(d, k, v)
        return d

    def ws(d):
        n = sz(0)
        return lib.hsv_verify_workspace_bytes(ctypes.byref(d), ctypes.byref(n)), n.value

    statuses = set(range(7))
    big = 2**31 - 1
    pick = lambda *xs: rng.choice(xs)
    # 1. random descriptors through the workspace query
    for _ in range(20000):
        d = desc(batch=pick(0, 1, 2, 16, 64, 65, 4096, big, -1),
                 n_draft=pick(0, 1, 8, 64, 65, 256, 257, big, -3),
                 n_q_heads=pick(1, 4, 8, 32, 30, 128, big, 0),
                 n_kv_heads=pick(1, 2, 8, 0, big, -2),
                 head_dim=pick(64, 128, 96, 0, 256, big),
                 kv_capacity=pick(0, 64, 4096, 32832, 196672, big, -5),
                 max_ctx=pick(0, 1, 31, 4000, 32768, 131072, big, -1),
                 n_sel=pick(0, 0, 1, 100, 4096, big, -1),
                 in_dtype=pick(0, 1, 7), out_dtype=pick(0, 1, 2),
                 scale=pick(0.0, 0.1, -1.0, float("nan"), float("inf")),
                 num_splits=pick(0, 0, 1, 7, 256, 257, -1, big),
                 flags=pick(0, 1, 2, 4, 6, 32, 64, 128, 0xFFFFFFFF),
                 block_size=pick(0, 0, 64, 128, 96, 16, 1 << 30, -64))
        code, n = ws(d)
        if code not in statuses:
            failures.append(f"workspace query returned {code}")
        elif code == m.HSV_OK and n == 0:
            failures.append("workspace query: OK with 0 bytes")
    # 2. selection workspace sizes
    for _ in range(5000):
        n = sz(0)
        code = lib.hsv_select_workspace_bytes(pick(0, 1, 8, 64, big, -1), pick(0, 1, 8, big, -1),
                                              pick(0, 1, 8192, 65544, 73728, 73729, 1 << 19,
                                                   (1 << 19) + 1, big, -1), ctypes.byref(n))
        if code not in statuses:
            failures.append(f"select workspace query returned {code}")
    # 3. entry points: missing pointers, malformed shapes, short workspaces
    d = desc()
    code, need = ws(d)
    ok_need = need if code == m.HSV_OK else 1 << 20
    expect = [
        (lib.hsv_verify_attn(ctypes.byref(d), None, fake, fake, fake, fake, None, fake, fake,
                             fake, sz(ok_need), None), m.HSV_ERR_NULL),
        (lib.hsv_verify_attn(ctypes.byref(d), fake, fake, fake, fake, fake, None, fake, fake,
                             fake, sz(100), None), m.HSV_ERR_WORKSPACE),
        (lib.hsv_verify_attn(None, fake, fake, fake, fake, fake, None, fake, fake, fake,
                             sz(ok_need), None), m.HSV_ERR_NULL),
        (lib.hsv_verify_attn_sparse(ctypes.byref(desc(n_sel=64)), fake, fake, fake, fake, fake,
                                    None, None, fake, fake, fake, sz(1 << 30), None),
         m.HSV_ERR_NULL),
        (lib.hsv_verify_attn_paged(ctypes.byref(desc(block_size=128, kv_capacity=32896)), fake, fake, fake, None,
                                   10, fake, fake, None, fake, fake, fake, sz(1 << 30), None),
         m.HSV_ERR_NULL),
        (lib.hsv_verify_attn_sparse_paged(ctypes.byref(desc(block_size=128, n_sel=64, n_draft=8, kv_capacity=32896)),
                                          fake, fake, fake, fake, 10, fake, fake, None, None,
                                          fake, fake, fake, sz(1 << 30), None), m.HSV_ERR_NULL),
        (lib.hsv_verify_attn_noalloc(ctypes.byref(desc(n_draft=300)), fake, fake, fake, fake,
                                     fake, None, fake, fake, None), m.HSV_ERR_SHAPE),
        (lib.hsv_tree_ancestor_mask(None, fake, 1, 8, None), m.HSV_ERR_NULL),
        (lib.hsv_tree_ancestor_mask(fake, fake, 1, 257, None), m.HSV_ERR_SHAPE),
        (lib.hsv_gather_kv(None, fake, fake, fake, fake, 1, 1, 64, 128, 8, m.HSV_BF16, None),
         m.HSV_ERR_NULL),
        (lib.hsv_lse_merge(None, fake, 2, 8, 128, fake, fake, m.HSV_F32, None), m.HSV_ERR_NULL),
        (lib.hsv_select_kv_idx(fake, fake, 1024, fake, 1, 1, 64, 4, 8, 16, None, fake, sz(1 << 20),
                               None), m.HSV_ERR_NULL),
        (lib.hsv_select_kv_idx(fake, fake, 1024, fake, 1, 1, 8, 4, 8, 16, fake, fake, sz(1 << 20),
                               None), m.HSV_ERR_SHAPE),
        (lib.hsv_tree_position_ids(None, fake, fake, 1, 8, None), m.HSV_ERR_NULL),
        (lib.hsv_accept_path(None, fake, fake, fake, fake, 1, 8, 64, 128, 8, m.HSV_BF16, None),
         m.HSV_ERR_NULL),
    ]
    for i, (got, want) in enumerate(expect):
        if got != want:
            failures.append(f"entry point case {i}: status {got}, expected {want}")
    for code in range(-1, 9):
        lib.hsv_status_string(code)
    if lib.hsv_version() < 1:
        failures.append("version")
    for f in failures[:20]:
        print(f, file=sys.stderr)
    if failures:
        print(f"{len(failures)} failure(s)", file=sys.stderr)
        return 1
    print("host driver: all cases passed")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
