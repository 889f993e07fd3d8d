"""The C ABI library without a GPU: it loads, exports every function that
the headers in include/ declare, and rejects bad arguments on the host before
touching the device."""
import ctypes
import os
import re

import pytest

import device_draft_verification_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(spec_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.LIB_PATH):
        pytest.fail("libspecverify.so is not built (run __graft_entry__.build())")
    return sv.load_library()


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("spec_verify_init", "spec_verify", "spec_accept_logprobs", "spec_verify_destroy",
              "spec_bandit_init", "spec_bandit_step", "spec_bandit_destroy"):
        assert n in names
    assert set(names) == set(sv.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_is_built_for_gfx950():
    data = open(sv.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_strerror(lib):
    assert sv.spec_verify_strerror(0) == "ok"
    assert sv.spec_verify_strerror(-1) == "invalid argument"
    assert sv.spec_verify_strerror(-77) == "unknown status"


def test_host_argument_checks(lib):
    h = ctypes.c_void_p()
    assert lib.spec_verify_init(4, 2, 100, 7, None, ctypes.byref(h)) == sv.binding.SPEC_EINVAL
    assert not h.value
    assert lib.spec_verify_init(-1, 2, 100, 1, None, ctypes.byref(h)) == sv.binding.SPEC_EINVAL
    # no offset word, or a misaligned one: refused before the context is used
    assert lib.spec_verify_offset_ptr(None, None, None, None, None, 0, None, None,
                                      None) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_offset_ptr(None, None, None, None, None, 0, ctypes.c_void_p(4),
                                      None, None) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_init(4, -1, 100, 1, None, ctypes.byref(h)) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_init(4, 2, 0, 1, None, ctypes.byref(h)) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_init(4, 2, 10, 1, None, None) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify(None, None, None, None, None, 0, 0, None, None) == sv.binding.SPEC_EINVAL
    assert lib.spec_accept_logprobs(None, None, 0, 0, None) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_copy_lse(None, None) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_destroy(None) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_enable_timing(None, 4) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_get_geometry(None, None) == sv.binding.SPEC_EINVAL
    assert lib.spec_verify_outcomes(None, None, None, None, 4, None, None, None, None) == \
        sv.binding.SPEC_EINVAL


def test_bandit_host_argument_checks(lib):
    E = sv.binding.SPEC_EINVAL
    h = ctypes.c_void_p()
    assert lib.spec_bandit_init(1, 3, 8, 4, 0, None, None) == E
    assert lib.spec_bandit_init(0, 3, 8, 4, 0, None, ctypes.byref(h)) == E  # no groups
    assert lib.spec_bandit_init(1, 0, 8, 4, 0, None, ctypes.byref(h)) == E  # no arms
    assert lib.spec_bandit_init(1, 65, 8, 4, 0, None, ctypes.byref(h)) == E  # > 64 arms
    assert lib.spec_bandit_init(3, 3, 8, 4, 0, None, ctypes.byref(h)) == E  # 8 % 3 != 0
    assert lib.spec_bandit_init(1, 3, 8, 0, 0, None, ctypes.byref(h)) == E  # gamma 0
    assert lib.spec_bandit_init(1, 3, 8, 4, 2, None, ctypes.byref(h)) == E  # policy
    assert not h.value
    assert lib.spec_bandit_step(None, None, None, 0, 0, None) == E
    assert lib.spec_bandit_get_state(None, None, None) == E
    assert lib.spec_bandit_set_state(None, None, None) == E
    assert lib.spec_bandit_set_stream(None, None) == E
    assert lib.spec_bandit_destroy(None) == E


def test_head_host_argument_checks(lib):
    E = sv.binding.SPEC_EINVAL
    h = ctypes.c_void_p()
    assert lib.spec_lowrank_head_init(8, 128, 64, 296, None, None) == E
    assert lib.spec_lowrank_head_init(0, 128, 64, 296, None, ctypes.byref(h)) == E   # no rows
    assert lib.spec_lowrank_head_init(8, 96, 64, 296, None, ctypes.byref(h)) == E    # d % 64
    assert lib.spec_lowrank_head_init(8, 128, 32, 296, None, ctypes.byref(h)) == E   # r % 64
    assert lib.spec_lowrank_head_init(8, 128, 64, 300, None, ctypes.byref(h)) == E   # V % 8
    assert not h.value
    assert lib.spec_lowrank_head(None, None, None, None, None, None, None) == E
    assert lib.spec_lowrank_head_copy_activation(None, None) == E
    assert lib.spec_lowrank_head_set_stream(None, None) == E
    assert lib.spec_lowrank_head_destroy(None) == E


def test_tree_host_argument_checks(lib):
    E = sv.binding.SPEC_EINVAL
    D = ctypes.c_double
    assert lib.spec_tree_prune(2, 0, None, None, D(0.0), 4, None, None, None, None, None) == E
    assert lib.spec_tree_prune(2, 257, None, None, D(0.0), 4, None, None, None, None, None) == E
    assert lib.spec_tree_prune(2, 8, None, None, D(0.5), 4, None, None, None, None, None) == E
    assert lib.spec_tree_prune(2, 8, None, None, D(0.0), 0, None, None, None, None, None) == E
    assert lib.spec_tree_prune(2, 8, None, None, D(0.0), 4, None, None, None, None, None) == E
    h = ctypes.c_void_p()
    assert lib.spec_tree_verify_init(2, 300, 100, 1, None, ctypes.byref(h)) == E
    assert lib.spec_tree_verify_init(2, 8, 100, 5, None, ctypes.byref(h)) == E
    assert not h.value
    assert lib.spec_tree_verify_greedy(None, None, None, None, None, None, None, None) == E
    assert lib.spec_tree_verify_sample(None, None, None, None, None, None, None, 0, 0, None, None,
                                       None) == E
    assert lib.spec_tree_verify_destroy(None) == E


def test_fanout_host_argument_checks(lib):
    E = sv.binding.SPEC_EINVAL
    V = ctypes.c_void_p
    ok = V(256)
    # lengths, list length, budget, batch
    assert lib.spec_outcome_fanout(2, 0, 16, ok, ok, 4, ok, None, None) == E
    assert lib.spec_outcome_fanout(2, 257, 16, ok, ok, 4, ok, None, None) == E
    assert lib.spec_outcome_fanout(2, 9, 0, ok, ok, 4, ok, None, None) == E
    assert lib.spec_outcome_fanout(2, 9, 65, ok, ok, 4, ok, None, None) == E
    assert lib.spec_outcome_fanout(2, 9, 16, ok, ok, -1, ok, None, None) == E
    assert lib.spec_outcome_fanout(-1, 9, 16, ok, ok, 4, ok, None, None) == E
    # missing or misaligned pointers
    assert lib.spec_outcome_fanout(2, 9, 16, None, ok, 4, ok, None, None) == E
    assert lib.spec_outcome_fanout(2, 9, 16, ok, None, 4, ok, None, None) == E
    assert lib.spec_outcome_fanout(2, 9, 16, ok, ok, 4, None, None, None) == E
    assert lib.spec_outcome_fanout(2, 9, 16, V(258), ok, 4, ok, None, None) == E
    assert lib.spec_outcome_fanout(2, 9, 16, ok, ok, 4, ok, V(260), None) == E
    # an empty batch launches nothing
    assert lib.spec_outcome_fanout(0, 9, 16, None, None, 4, None, None, None) == 0


def test_binding_refuses_missing_library(tmp_path, lib):
    saved = sv.binding._lib
    sv.binding._lib = None
    try:
        with pytest.raises(RuntimeError):
            sv.binding.load_library(str(tmp_path / "missing.so"))
    finally:
        sv.binding._lib = saved


def test_noalloc_host_checks(lib):
    """spec_verify_noalloc refuses bad shapes and pointers, and a shape whose
    workspace exceeds its fixed scratch array, on the host before any HIP call
    (so this runs without a GPU: the pointers are never dereferenced)."""
    E, X = sv.binding.SPEC_EINVAL, sv.binding.SPEC_ESCRATCH
    p = ctypes.c_void_p(1 << 20)  # aligned stand-in, never touched
    args = (p, p, p, p, 0, 0, p, p)
    assert lib.spec_verify_noalloc(4, 2, 100, 7, None, *args) == E          # dtype
    assert lib.spec_verify_noalloc(4, -1, 100, 1, None, *args) == E         # gamma
    assert lib.spec_verify_noalloc(4, 2, 0, 1, None, *args) == E            # vocab
    assert lib.spec_verify_noalloc(4, 2, 100, 1, None, p, None, p, p, 0, 0, p, p) == E
    assert lib.spec_verify_noalloc(4, 2, 100, 1, None, p, p, p, p, 0, 0, ctypes.c_void_p(2), p) == E
    assert lib.spec_verify_noalloc(0, 2, 100, 1, None, None, None, None, None, 0, 0, None,
                                   None) == sv.binding.SPEC_OK            # empty batch
    # two-kernel draw (B < 128): 127 * ceil(V / 64) tile sums exceed 16 MiB
    assert lib.spec_verify_noalloc(127, 1, 1 << 25, 1, None, *args) == X
    assert sv.spec_verify_strerror(X).startswith("the shape's workspace")


def test_tree_status_hooks_refuse_null(lib):
    E = sv.binding.SPEC_EINVAL
    n = ctypes.c_uint64(0)
    assert lib.spec_tree_verify_gave_up(None, ctypes.byref(n)) == E
    assert lib.spec_tree_verify_set_spin_limit(None, 4) == E


def test_probe_host_checks(lib):
    E = sv.binding.SPEC_EINVAL
    p = ctypes.c_void_p(1 << 20)
    assert lib.spec_hbm_read_probe(None, 1024, p, 4, None) == E
    assert lib.spec_hbm_read_probe(p, 1000, p, 4, None) == E       # not a multiple of 16
    assert lib.spec_hbm_read_probe(p, 1024, p, 0, None) == E       # no workgroups
    assert lib.spec_hbm_read_probe(p, 0, p, 4, None) == sv.binding.SPEC_OK
