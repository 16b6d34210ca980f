"""The C-ABI library loads, exports what include/sparse_kv.h declares, and
rejects bad host-visible arguments before queuing anything (CPU only: no
call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_kv.h")


@pytest.fixture(scope="module")
def skv():
    import sparse_kv_amd

    if not os.path.exists(sparse_kv_amd.LIB_PATH):
        from sparse_kv_amd import build

        build.build()
    sparse_kv_amd.lib()
    return sparse_kv_amd


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\*?(attn_[a-z_]+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(skv):
    names = declared_functions()
    assert len(names) >= 10, names
    lib = ctypes.CDLL(skv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(skv.EXPORTS)


def dims(**kw):
    from sparse_kv_amd import AttnDims

    d = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=64, max_blocks=4, dtype=1, scale=0.1)
    d.update(kw)
    return AttnDims(**d)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


@pytest.mark.parametrize("kw,expect", [
    (dict(head_dim=96), -2), (dict(head_dim=0), -1), (dict(block_size=32), -2),
    (dict(num_q_heads=7), -1), (dict(num_q_heads=32, num_kv_heads=2), -2), (dict(dtype=5), -1),
    (dict(max_blocks=0), -1), (dict(batch=-1), -1), (dict(scale=float("nan")), -1),
    (dict(max_blocks=1 << 20), -2),
])
def test_dims_validation(skv, kw, expect):
    lib = skv.lib()
    d = dims(**kw)
    st = lib.attn_decode_dense(ctypes.byref(d), FAKE, FAKE, FAKE, None, 0, -1, 4, FAKE, FAKE, FAKE, None)
    assert st == expect


def test_argument_validation(skv):
    lib = skv.lib()
    d = dims()
    assert lib.attn_decode_dense(None, FAKE, FAKE, FAKE, None, 0, -1, 4, FAKE, FAKE, FAKE, None) == -1
    assert lib.attn_decode_dense(ctypes.byref(d), None, FAKE, FAKE, None, 0, -1, 4, FAKE, FAKE, FAKE, None) == -1
    assert lib.attn_decode_dense(ctypes.byref(d), FAKE, FAKE, FAKE, None, 0, -1, 0, FAKE, FAKE, FAKE, None) == -1
    assert lib.attn_decode_dense(ctypes.byref(d), FAKE, FAKE, FAKE, None, -1, -1, 4, FAKE, FAKE, FAKE, None) == -1
    assert lib.attn_merge_states(4, 0, 128, FAKE, FAKE, FAKE, FAKE, None, None, None) == -1
    assert lib.attn_merge_states(4, 2, 96, FAKE, FAKE, FAKE, FAKE, None, None, None) == -2
    assert lib.attn_merge_states(4, 2, 128, None, FAKE, FAKE, FAKE, None, None, None) == -1
    # top-k: k > 0 needs scores; max_sel must hold the forced blocks plus k
    assert lib.attn_select_topk(ctypes.byref(d), None, None, 2, 1, 1, 4, FAKE, FAKE, None) == -1
    assert lib.attn_select_topk(ctypes.byref(d), FAKE, None, 2, 1, 1, 3, FAKE, FAKE, None) == -1
    assert lib.attn_select_topk(ctypes.byref(d), FAKE, None, -1, 1, 1, 4, FAKE, FAKE, None) == -1
    assert lib.attn_decode_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, 4, 2, FAKE, FAKE, FAKE,
                                  None) == -1
    # ART: patience >= 1, probe_dim in [0, 16], thresholds not NaN
    args = [FAKE, FAKE, FAKE, None, None]
    assert lib.attn_decode_art(ctypes.byref(d), *args, 1e-3, 1e-4, 0, 8, FAKE, FAKE, None, None) == -1
    assert lib.attn_decode_art(ctypes.byref(d), *args, 1e-3, 1e-4, 2, -1, FAKE, FAKE, None, None) == -1
    assert lib.attn_decode_art(ctypes.byref(d), *args, 1e-3, 1e-4, 2, 17, FAKE, FAKE, None, None) == -2
    assert lib.attn_decode_art(ctypes.byref(d), *args, float("nan"), 1e-4, 2, 8, FAKE, FAKE, None, None) == -1
    assert lib.attn_decode_art(ctypes.byref(d), *args, 1e-3, 1e-4, 2, 8, None, FAKE, None, None) == -1
    # ART over a list: the list, its counts and max_list >= 1 are required
    lst = [FAKE, FAKE, FAKE, None]
    assert lib.attn_decode_art_list(ctypes.byref(d), *lst, None, FAKE, 4, 1e-3, 1e-4, 2, 8, FAKE, FAKE, None,
                                    None) == -1
    assert lib.attn_decode_art_list(ctypes.byref(d), *lst, FAKE, None, 4, 1e-3, 1e-4, 2, 8, FAKE, FAKE, None,
                                    None) == -1
    assert lib.attn_decode_art_list(ctypes.byref(d), *lst, FAKE, FAKE, 0, 1e-3, 1e-4, 2, 8, FAKE, FAKE, None,
                                    None) == -1
    assert lib.attn_decode_art_list(ctypes.byref(d), *lst, FAKE, FAKE, 4, 1e-3, 1e-4, 0, 8, FAKE, FAKE, None,
                                    None) == -1
    # centroid update: k, centroids and span_hint >= 1 are required
    assert lib.attn_update_centroids(ctypes.byref(d), None, None, None, 1, FAKE, None) == -1
    assert lib.attn_update_centroids(ctypes.byref(d), FAKE, None, None, 1, None, None) == -1
    assert lib.attn_update_centroids(ctypes.byref(d), FAKE, None, None, 0, FAKE, None) == -1
    # two-level selection: group >= 1, capacity limits, max_sel as for top-k
    assert lib.attn_build_super_centroids(ctypes.byref(d), FAKE, None, 0, FAKE, None) == -1
    assert lib.attn_build_super_centroids(ctypes.byref(d), None, None, 4, FAKE, None) == -1
    tl = lambda dd, group, kc, k, ms: lib.attn_select_two_level(ctypes.byref(dd), FAKE, FAKE, FAKE, None, group, kc,
                                                                k, 1, 1, ms, FAKE, FAKE, None)
    assert tl(d, 0, 2, 2, 4) == -1
    assert tl(d, 2, 2, 2, 3) == -1  # max_sel below sink + window + k
    assert tl(d, 2, -1, 2, 4) == -1
    assert tl(dims(max_blocks=4097 * 2), 2, 1, 1, 4) == -2  # more than 4096 super-blocks
    assert tl(dims(max_blocks=16384), 16, 513, 1, 4) == -2  # 513 * 16 candidates
    assert tl(dims(batch=0, max_blocks=8192), 16, 512, 1, 4) == 0
    # paged cache descriptors: pools, a table of >= max_blocks entries per row, pool_blocks >= 1
    from sparse_kv_amd import AttnPagedKV

    good = AttnPagedKV(0x1000, 0x1000, 16, 0x1000, 4)
    for bad in (AttnPagedKV(None, 0x1000, 16, 0x1000, 4), AttnPagedKV(0x1000, None, 16, 0x1000, 4),
                AttnPagedKV(0x1000, 0x1000, 0, 0x1000, 4), AttnPagedKV(0x1000, 0x1000, 16, None, 4),
                AttnPagedKV(0x1000, 0x1000, 16, 0x1000, 3)):
        assert lib.attn_decode_dense_paged(ctypes.byref(d), FAKE, ctypes.byref(bad), None, 0, -1, 4, FAKE, FAKE, FAKE,
                                           None) == -1
    assert lib.attn_decode_dense_paged(ctypes.byref(d), FAKE, None, None, 0, -1, 4, FAKE, FAKE, FAKE, None) == -1
    assert lib.attn_decode_dense_paged(ctypes.byref(d), FAKE, ctypes.byref(good), None, 0, -1, 0, FAKE, FAKE, FAKE,
                                       None) == -1
    assert lib.attn_decode_sparse_paged(ctypes.byref(d), FAKE, ctypes.byref(good), None, None, FAKE, 4, 2, FAKE, FAKE,
                                        FAKE, None) == -1
    konly = AttnPagedKV(0x1000, None, 16, 0x1000, 4)  # centroids read K only
    assert lib.attn_build_centroids_paged(ctypes.byref(d), ctypes.byref(konly), None, None, None) == -1
    assert lib.attn_update_centroids_paged(ctypes.byref(d), ctypes.byref(konly), None, None, 0, FAKE, None) == -1
    assert lib.attn_decode_art_paged(ctypes.byref(d), FAKE, ctypes.byref(konly), None, None, 1e-3, 1e-4, 2, 8, FAKE,
                                     FAKE, None, None) == -1
    assert lib.attn_decode_art_paged(ctypes.byref(d), FAKE, ctypes.byref(good), None, None, 1e-3, 1e-4, 0, 8, FAKE,
                                     FAKE, None, None) == -1
    d0 = dims(batch=0)
    assert lib.attn_decode_dense_paged(ctypes.byref(d0), FAKE, ctypes.byref(good), None, 0, -1, 4, FAKE, FAKE, FAKE,
                                       None) == 0
    # importance order: scores and order are required; at most 16384 blocks after the sink
    assert lib.attn_order_blocks(ctypes.byref(d), None, None, FAKE, None) == -1
    assert lib.attn_order_blocks(ctypes.byref(d), FAKE, None, None, None) == -1
    assert lib.attn_order_blocks(ctypes.byref(dims(max_blocks=16386)), FAKE, None, FAKE, None) == -2
    assert lib.attn_order_blocks(ctypes.byref(dims(batch=0, max_blocks=16385)), FAKE, None, FAKE, None) == 0
    # empty batch is a no-op success
    d0 = dims(batch=0)
    assert lib.attn_decode_dense(ctypes.byref(d0), FAKE, FAKE, FAKE, None, 0, -1, 4, FAKE, FAKE, FAKE, None) == 0


def test_routed_workspace_and_validation(skv):
    lib = skv.lib()
    d = dims()
    small = lib.attn_routed_workspace_bytes(ctypes.byref(d), 8, 2, 4)
    big = lib.attn_routed_workspace_bytes(ctypes.byref(d), 8, 4, 4)
    assert 0 < small < big
    assert lib.attn_routed_workspace_bytes(ctypes.byref(d), 0, 2, 4) == 0
    assert lib.attn_routed_workspace_bytes(ctypes.byref(dims(head_dim=96)), 8, 2, 4) == 0
    mask = (ctypes.c_uint8 * 2)(1, 0)
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    P = ctypes.c_void_p
    call = lambda ws_bytes, sa=FAKE: lib.attn_decode_routed(
        ctypes.byref(d), 2, ctypes.cast(mask, P), ctypes.cast(ptrs, P), ctypes.cast(ptrs, P), ctypes.cast(ptrs, P),
        None, 8, 2, sa, FAKE, 4, 4, FAKE, ws_bytes, ctypes.cast(ptrs, P), None)
    assert call(small - 1) == -4
    assert call(small, sa=None) == -1  # a sparse layer needs its block list
    big_sa = lib.attn_decode_routed(ctypes.byref(d), 2, ctypes.cast(mask, P), ctypes.cast(ptrs, P),
                                    ctypes.cast(ptrs, P), ctypes.cast(ptrs, P), None, 8, 2, FAKE, FAKE, 4,
                                    (1 << 24) + 1, FAKE, 1 << 40, ctypes.cast(ptrs, P), None)
    assert big_sa == -1  # split counts are bounded
    # the workspace-free variant: the same checks, then the states must fit its static scratch
    stat = lambda dd, ns, sps, sas, sa=FAKE, n=2: lib.attn_decode_routed_static(
        ctypes.byref(dd), n, ctypes.cast(mask, P), ctypes.cast(ptrs, P), ctypes.cast(ptrs, P), ctypes.cast(ptrs, P),
        None, ns, sps, sa, FAKE, 4, sas, ctypes.cast(ptrs, P), None)
    assert stat(d, 8, 2, 4, sa=None) == -1
    assert stat(d, 0, 2, 4) == -1
    assert stat(dims(head_dim=96), 8, 2, 4) == -2
    big_d = dims(batch=64, num_q_heads=32, num_kv_heads=8)
    assert lib.attn_routed_workspace_bytes(ctypes.byref(big_d), 8, 4, 4) > skv.ROUTED_STATIC_BYTES
    assert stat(big_d, 8, 4, 4) == -4  # refused before anything touches a device
    assert stat(dims(batch=0), 8, 2, 4) == 0
    assert stat(d, 8, 2, 4, n=0) == 0


def test_art_workspace_and_validation(skv):
    lib = skv.lib()
    d = dims()  # B = 2, Hkv = 2, G = 4, d = 128
    per_unit_g4 = lib.attn_art_workspace_bytes(ctypes.byref(d)) // 4
    assert per_unit_g4 > 0 and per_unit_g4 * 4 == lib.attn_art_workspace_bytes(ctypes.byref(d))
    # the ring holds fp32 states: twice the query heads per slot, twice the bytes
    per_unit_g8 = lib.attn_art_workspace_bytes(ctypes.byref(dims(num_q_heads=16))) // 4
    assert 1.9 < per_unit_g8 / per_unit_g4 < 2.1
    assert lib.attn_art_workspace_bytes(ctypes.byref(dims(head_dim=64))) < 4 * per_unit_g4
    assert lib.attn_art_workspace_bytes(ctypes.byref(dims(batch=64))) == 128 * per_unit_g4
    assert lib.attn_art_workspace_bytes(ctypes.byref(dims(batch=65))) == 0  # beyond 128 units: none used
    assert lib.attn_art_workspace_bytes(ctypes.byref(dims(batch=0))) == 0
    assert lib.attn_art_workspace_bytes(ctypes.byref(dims(head_dim=96))) == 0
    assert lib.attn_art_workspace_bytes(None) == 0
    need = lib.attn_art_workspace_bytes(ctypes.byref(d))
    args = (FAKE, FAKE, FAKE, None, None, 1e-3, 1e-4, 2, 8)
    call = lambda ws, nbytes, dd=d: lib.attn_decode_art_ws(ctypes.byref(dd), *args, ws, nbytes, FAKE, FAKE, None,
                                                           None)
    assert call(None, need) == -1       # a needed workspace is missing
    assert call(FAKE, need - 1) == -4   # too small
    assert lib.attn_decode_art_ws(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, 1e-3, 1e-4, 0, 8, FAKE, need,
                                  FAKE, FAKE, None, None) == -1  # the attn_decode_art checks still apply
    assert call(None, 0, dims(head_dim=96)) == -2
    assert call(None, 0, dims(batch=0)) == 0  # nothing to do, nothing needed
    # the list and paged twins check the workspace the same way, then their own arguments
    lst = (FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 1e-3, 1e-4, 2, 8)
    assert lib.attn_decode_art_list_ws(ctypes.byref(d), *lst, None, need, FAKE, FAKE, None, None) == -1
    assert lib.attn_decode_art_list_ws(ctypes.byref(d), *lst, FAKE, need - 1, FAKE, FAKE, None, None) == -4
    assert lib.attn_decode_art_list_ws(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, FAKE, 4, 1e-3, 1e-4, 2, 8,
                                       FAKE, need, FAKE, FAKE, None, None) == -1  # no block list
    from sparse_kv_amd import AttnPagedKV

    kv = AttnPagedKV(k_pool=0x1000, v_pool=None, pool_blocks=8, block_table=0x1000, table_stride=4)
    pg = (FAKE, ctypes.byref(kv), None, None, 1e-3, 1e-4, 2, 8)
    assert lib.attn_decode_art_paged_ws(ctypes.byref(d), *pg, FAKE, need - 1, FAKE, FAKE, None, None) == -4
    assert lib.attn_decode_art_paged_ws(ctypes.byref(d), *pg, FAKE, need, FAKE, FAKE, None, None) == -1  # no v pool


def test_status_strings(skv):
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(skv.attn_status_string(code), str) and skv.attn_status_string(code)


def test_header_is_plain_c_and_links(skv, tmp_path):
    """include/sparse_kv.h compiles as C99 and a C program linked against the
    library gets the documented status codes (validation paths only)."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = os.path.join(ROOT, "tests", "c", "abi_from_c.c")
    exe = str(tmp_path / "abi_from_c")
    libdir = os.path.dirname(skv.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    src, "-o", exe, "-L", libdir, "-lsparse_kv", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
