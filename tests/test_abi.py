"""The C-ABI library on the CPU: it loads, exports every entry point the headers declare,
and rejects bad host-side arguments before touching the GPU."""

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECL = re.compile(r"^(?:const\s+)?(?:spec_status_t|size_t|int|int64_t|char|void)\s*\*?\s*(\w+)\s*\(", re.M)


def declared_functions():
    names = []
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        with open(h) as f:
            names += DECL.findall(f.read())
    return names


@pytest.fixture(scope="module")
def lib():
    from draft_token_verification_09_amd.build import library_path

    path = library_path()
    if not os.path.exists(path):
        pytest.fail(f"{path} not built: run python -m draft_token_verification_09_amd.build")
    from draft_token_verification_09_amd import binding

    return binding.lib()


def test_headers_declare_the_three_operations():
    names = declared_functions()
    for n in ("spec_verify_chain", "spec_verify_tree_greedy", "ngram_propose", "spec_verify_chain_workspace_size",
              "spec_verify_tree_greedy_workspace_size", "spec_status_string", "spec_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.spec_status_string(0) == b"SPEC_OK"
    assert lib.spec_status_string(3) == b"SPEC_ERR_WORKSPACE"


def test_workspace_sizes_are_host_only(lib):
    assert lib.spec_verify_chain_workspace_size(64, 5, 128256, 1) > 0
    assert lib.spec_verify_chain_workspace_size(0, 5, 128256, 1) == 0
    assert lib.spec_verify_chain_workspace_size(4, 65, 100, 1) == 0
    assert lib.spec_verify_tree_greedy_workspace_size(32, 61, 128256, 1) > 0
    assert lib.spec_verify_tree_greedy_workspace_size(1, 2000, 100, 1) == 0


def test_host_argument_errors_return_before_any_launch(lib):
    null = None
    # K = 0
    st = lib.spec_verify_chain(null, null, 1, null, null, null, null, null, 2, 0, 10,
                               null, null, null, null, null, null, 0, null)
    assert st == 1 and b"K >= 1" in lib.spec_last_error()
    # K too large
    st = lib.spec_verify_chain(null, null, 1, null, null, null, null, null, 2, 65, 10,
                               null, null, null, null, null, null, 0, null)
    assert st == 2
    # unknown dtype
    st = lib.spec_verify_chain(null, null, 7, null, null, null, null, null, 2, 5, 10,
                               null, null, null, null, null, null, 0, null)
    assert st == 1
    # required pointers missing
    st = lib.spec_verify_chain(null, null, 1, null, null, null, null, null, 2, 5, 10,
                               null, null, null, null, null, null, 0, null)
    assert st == 1
    # packed without offsets
    fake = ctypes.c_void_p(1 << 20)
    st = lib.spec_verify_chain(fake, null, 1, fake, null, fake, fake, fake, 2, 5, 10,
                               fake, fake, null, fake, null, null, 0, null)
    assert st == 1
    # workspace missing / too small / misaligned
    st = lib.spec_verify_chain(fake, null, 1, fake, null, fake, fake, fake, 2, 5, 10,
                               fake, fake, null, null, null, null, 0, null)
    assert st == 3
    st = lib.spec_verify_chain(fake, null, 1, fake, null, fake, fake, fake, 2, 5, 10,
                               fake, fake, null, null, null, ctypes.c_void_p(1 << 20), 16, null)
    assert st == 3
    st = lib.spec_verify_chain(fake, null, 1, fake, null, fake, fake, fake, 2, 5, 10,
                               fake, fake, null, null, null, ctypes.c_void_p((1 << 20) + 8), 1 << 20, null)
    assert st == 3
    # tree: too many nodes; max_depth beyond N1
    st = lib.spec_verify_tree_greedy(null, 1, null, null, 1, 2000, 10, 3, null, null, null, null, null, 0, null)
    assert st == 2
    st = lib.spec_verify_tree_greedy(null, 1, null, null, 1, 4, 10, 9, null, null, null, null, null, 0, null)
    assert st == 1
    # n-gram: n_min > n_max, n_max too large
    assert lib.ngram_propose(null, null, 1, 10, 3, 2, 5, null, null, null, null) == 1
    assert lib.ngram_propose(null, null, 1, 10, 1, 17, 5, null, null, null, null) == 2


def test_empty_batches_need_no_gpu_work(lib):
    null = None
    assert lib.spec_verify_tree_greedy(null, 1, null, null, 0, 4, 10, 3, null, null, null, null, null, 0, null) == 0
    assert lib.ngram_propose(null, null, 0, 10, 1, 4, 5, null, null, null, null) == 0


def test_mask_and_commit_host_errors(lib):
    null = None
    fake = ctypes.c_void_p(1 << 20)
    # mask: too many nodes, no outputs, N1 = 0
    assert lib.spec_tree_mask(fake, 1, 2000, fake, null, null) == 2
    assert lib.spec_tree_mask(fake, 1, 5, null, null, null) == 1
    assert lib.spec_tree_mask(fake, 1, 0, fake, null, null) == 1
    assert lib.spec_tree_mask(null, 0, 5, null, null, null) == 0
    # commit: entry not a multiple of 16 bytes, bad path stride, plane stride too small,
    # misaligned buffers, NULL lengths
    args = dict(kv=fake, path=fake, P=7, acc=fake, clen=fake, B=4, N1=61, L=32, planes=2, eb=2048,
                sp=4 * 61 * 2048, dp=4 * 32 * 2048, cache=ctypes.c_void_p(1 << 21), out=null)

    def commit(**kw):
        a = dict(args, **kw)
        return lib.spec_commit_path(a["kv"], a["path"], a["P"], a["acc"], a["clen"], a["B"], a["N1"], a["L"],
                                    a["planes"], a["eb"], a["sp"], a["dp"], a["cache"], a["out"], null)

    assert commit(eb=24) == 1
    assert commit(P=0) == 1
    assert commit(P=2000) == 1
    assert commit(sp=100) == 1
    assert b"plane stride" in lib.spec_last_error()
    assert commit(dp=4 * 32 * 2048 - 16) == 1
    assert commit(kv=ctypes.c_void_p((1 << 20) + 8)) == 1
    assert commit(clen=null) == 1
    assert commit(B=0) == 0


def test_knobs_set_get_and_restore(lib):
    from draft_token_verification_09_amd import binding as bd

    assert bd.spec_get_knob(bd.SPEC_KNOB_CHUNK_VECTORS) == 0
    assert bd.spec_get_knob(bd.SPEC_KNOB_POLL_LIMIT) == 1 << 18
    with bd.knob(bd.SPEC_KNOB_CHUNK_VECTORS, 4), bd.knob(bd.SPEC_KNOB_POLL_LIMIT, 0):
        assert bd.spec_get_knob(bd.SPEC_KNOB_CHUNK_VECTORS) == 4
        assert bd.spec_get_knob(bd.SPEC_KNOB_POLL_LIMIT) == 0
    assert bd.spec_get_knob(bd.SPEC_KNOB_CHUNK_VECTORS) == 0
    assert bd.spec_get_knob(bd.SPEC_KNOB_POLL_LIMIT) == 1 << 18
    with pytest.raises(bd.SpecError):
        bd.spec_set_knob(bd.SPEC_KNOB_CHUNK_VECTORS, 3)  # not a chunk size
    with pytest.raises(bd.SpecError):
        bd.spec_set_knob(7, 1)  # no such knob
    assert lib.spec_get_knob(7) == -1
    bd.spec_set_knob(bd.SPEC_KNOB_POLL_LIMIT, 5)
    bd.spec_set_knob(bd.SPEC_KNOB_POLL_LIMIT, -1)  # negative: back to the default
    assert bd.spec_get_knob(bd.SPEC_KNOB_POLL_LIMIT) == 1 << 18
    assert bd.spec_get_knob(bd.SPEC_KNOB_SINGLE_LAUNCH) == 0
    with bd.knob(bd.SPEC_KNOB_SINGLE_LAUNCH, 1):
        assert bd.spec_get_knob(bd.SPEC_KNOB_SINGLE_LAUNCH) == 1
    assert bd.spec_get_knob(bd.SPEC_KNOB_SINGLE_LAUNCH) == 0
    with pytest.raises(bd.SpecError):
        bd.spec_set_knob(bd.SPEC_KNOB_SINGLE_LAUNCH, 2)  # only 0 and 1
    assert bd.spec_get_knob(bd.SPEC_KNOB_XCD_LOCAL) == 1
    with bd.knob(bd.SPEC_KNOB_XCD_LOCAL, 0):
        assert bd.spec_get_knob(bd.SPEC_KNOB_XCD_LOCAL) == 0
    assert bd.spec_get_knob(bd.SPEC_KNOB_XCD_LOCAL) == 1
    with pytest.raises(bd.SpecError):
        bd.spec_set_knob(bd.SPEC_KNOB_XCD_LOCAL, 2)  # only 0 and 1


def test_workspace_size_covers_the_single_launch_layout(lib):
    # a shape that may run as one launch needs room for its hand-over words on top of the
    # separate launches' regions; the size must not depend on whether the single launch is
    # allowed when it is asked, since a call may be made with the other setting
    from draft_token_verification_09_amd import binding as bd

    small = bd.spec_verify_chain_workspace_size(1, 5, 32000, 0)
    with bd.knob(bd.SPEC_KNOB_SINGLE_LAUNCH, 1):
        assert bd.spec_verify_chain_workspace_size(1, 5, 32000, 0) == small
    # at least the single launch's tagged partial words: 3 words for each of 11 rows x 8 chunks x 4 waves
    assert small >= 3 * 8 * 11 * 8 * 4


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    # host-side: the allocation-free chain call checks the scratch its shape needs against the
    # library's 16 MiB array before it looks at any pointer or launches anything
    B, K, V = 4096, 8, 152064
    assert lib.spec_verify_chain_workspace_size(B, K, V, 1) > 16 << 20
    st = lib.spec_verify_chain_noalloc(1, 1, 1, 1, None, 1, 1, 1, B, K, V, 1, 1, None, None, None, None)
    assert st == 2  # SPEC_ERR_UNSUPPORTED
    assert b"allocation-free" in lib.spec_last_error()
