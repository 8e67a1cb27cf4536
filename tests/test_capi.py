"""The C ABI library loads, exports every function include/pst.h declares,
and rejects bad arguments before any HIP call (CPU only: no call here
reaches the GPU)."""

import ctypes

import pytest

import prefix_shared_tree_packed_amd as pst
from prefix_shared_tree_packed_amd import _lib


def test_exports_every_declared_function():
    lib = pst.load()
    names = pst.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib._SIGS), "binding and header disagree"


def test_library_built_from_the_sources_in_the_tree(tmp_path):
    """The in-tree library records the digest of the sources it was built
    from, equal to that of the sources at hand (a stale build would have
    been refused by load()); a digest that differs is refused, and an edit
    to any source changes the digest."""
    from prefix_shared_tree_packed_amd import build
    lib = pst.load()
    want = build.sources_sha256()
    assert lib.pst_build_sources_sha256().decode() == want
    _lib.verify_build(lib, want)
    with pytest.raises(RuntimeError, match="other sources"):
        _lib.verify_build(lib, "0" * 64)
    # the same sources elsewhere give the same digest; one byte more does not
    import os
    import shutil
    pkg = os.path.basename(build.PKG)
    shutil.copytree(build.CSRC, tmp_path / pkg / "csrc", ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(build.PKG, "build.py"), tmp_path / pkg / "build.py")
    shutil.copytree(build.INCLUDE, tmp_path / "include")
    assert build.sources_sha256(str(tmp_path)) == want
    with open(tmp_path / pkg / "csrc" / "kernels" / "common.h", "ab") as f:
        f.write(b"\n")
    assert build.sources_sha256(str(tmp_path)) != want


def test_device_entry_points_reject_null_meta():
    lib = pst.load()
    p = ctypes.c_void_p(16)
    rc = lib.pst_tree_attn_fwd(p, p, p, p, p, None, 32, 8, 128, 1, 0.0, None)
    assert _lib.ERRORS[rc] == "PST_EINVAL"
    rc = lib.pst_gather_tree_logprobs_entropy(p, 100, 1, None, p, p, None, None)
    assert _lib.ERRORS[rc] == "PST_EINVAL"
    rc = lib.pst_tree_attn_bwd(p, p, p, p, p, p, p, p, p, p, 0, None, 32, 8, 128, 1, 0.0, None)
    assert _lib.ERRORS[rc] == "PST_EINVAL"
    assert b"NULL" in lib.pst_last_error()
    rc = lib.pst_tree_attn_bwd_noalloc(p, p, p, p, p, p, p, p, p, None, 32, 8, 128, 1, 0.0, None)
    assert _lib.ERRORS[rc] == "PST_EINVAL"
    rc = lib.pst_gather_tree_logprobs_entropy_bwd(p, 100, 1, None, p, p, None, p, None)
    assert _lib.ERRORS[rc] == "PST_EINVAL"
    rc = lib.pst_tree_rope(p, None, 8, 128, 1, 0.0, 0, None)
    assert _lib.ERRORS[rc] == "PST_EINVAL"
    rc = lib.pst_tree_dense_mask(None, 0, p, None)
    assert _lib.ERRORS[rc] == "PST_EINVAL"
    rc = lib.pst_forest_meta_update(None, None, None)
    assert _lib.ERRORS[rc] == "PST_EINVAL"


def test_build_rejects_unknown_flags():
    import numpy as np
    lib = pst.load()
    toks = np.array([1, 2, 3], dtype=np.int32)
    offs = np.array([0, 3], dtype=np.int64)
    h = ctypes.c_void_p(1)
    rc = lib.pst_build_tree_ex(toks.ctypes.data_as(_lib.P32), offs.ctypes.data_as(_lib.P64), 1,
                               128, 2, ctypes.byref(h))
    assert _lib.ERRORS[rc] == "PST_EINVAL" and not h.value


def test_meta_create_rejects_bad_tree_index():
    f = pst.build_tree([[1, 2, 3]], 128)
    lib = pst.load()
    out = ctypes.c_void_p()
    for t in (-1, 1):
        rc = lib.pst_tree_meta_create(f._h, t, None, ctypes.byref(out))
        assert _lib.ERRORS[rc] == "PST_ERANGE"
        assert not out.value


def test_forest_meta_rejects_null_forest():
    lib = pst.load()
    out = ctypes.c_void_p()
    assert _lib.ERRORS[lib.pst_forest_meta_create(None, None, ctypes.byref(out))] == "PST_EINVAL"
    assert _lib.ERRORS[lib.pst_forest_meta_create(None, None, None)] == "PST_EINVAL"


def test_null_arguments():
    lib = pst.load()
    out = ctypes.c_void_p()
    assert _lib.ERRORS[lib.pst_build_tree(None, None, 1, 128, ctypes.byref(out))] == "PST_EINVAL"
    assert _lib.ERRORS[lib.pst_forest_num_trees(None, None)] == "PST_EINVAL"
    assert _lib.ERRORS[lib.pst_forest_stats(None, None)] == "PST_EINVAL"
    f = pst.build_tree([[1, 2, 3]], 128)
    with pytest.raises(pst.PstError):
        f.sizes(5)
