"""The C-ABI library loads and exports what include/specverify.h declares; host-side
argument checks and workspace queries work without a GPU (no compute calls)."""
import ctypes
import os
import re

import pytest

import accept_step_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:sv_status|int32_t|const char\s*\*)\s+(\w+)\s*\(", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.library_path()):
        pytest.fail("libspecverify.so is not built (run python -m accept_step_amd.build)")
    return sv.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"verify_forward", "spec_verify_greedy", "spec_verify_sample"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_version_and_status_strings(lib):
    assert lib.sv_version() == 10000
    assert lib.sv_status_string(0) == b"SV_OK"
    assert lib.sv_status_string(4) == b"SV_ERR_WORKSPACE"
    assert lib.sv_status_string(99) == b"SV_ERR_UNKNOWN"


def _model(vocab=1000, d=64, n_layers=0, wdtype=sv.SV_BF16):
    m = sv._SvModel()
    m.n_layers, m.vocab, m.d_model, m.wdtype = n_layers, vocab, d, wdtype
    m.lm_head = 0x10000            # never dereferenced by the host checks below
    return m


FAKE = ctypes.c_void_p(0x20000)     # 256-byte aligned stand-in pointer, never dereferenced


def greedy(lib, m, kind=sv.SV_IN_HIDDEN, inp=FAKE, B=1, gamma=4, draft=FAKE, ws=None, nbytes=0, diag=None):
    n = ctypes.c_size_t(nbytes)
    st = lib.spec_verify_greedy(ctypes.byref(m) if m is not None else None, kind, inp, B, gamma, draft, None,
                                FAKE, FAKE, None, diag, ws, ctypes.byref(n), None)
    return st, n.value


def test_argument_errors_are_reported_before_any_launch(lib):
    m = _model()
    assert greedy(lib, None)[0] == 1
    assert greedy(lib, m, inp=None)[0] == 1
    assert greedy(lib, m, B=0)[0] == 1
    assert greedy(lib, m, gamma=0)[0] == 1
    assert greedy(lib, m, gamma=16)[0] == 1
    assert b"gamma" in lib.sv_last_error()
    assert greedy(lib, m, draft=None)[0] == 1
    assert greedy(lib, _model(vocab=1))[0] == 1
    assert greedy(lib, _model(d=48))[0] == 3            # bf16 head needs d % 32 == 0
    assert greedy(lib, _model(wdtype=7))[0] == 2
    assert greedy(lib, m, kind=9)[0] == 1
    assert greedy(lib, _model(n_layers=1), kind=sv.SV_IN_HIDDEN)[0] == 1
    assert greedy(lib, m, kind=sv.SV_IN_TOKENS)[0] == 1  # no layers / cache


def test_sampling_argument_errors(lib):
    m = _model()

    def sample(T=1.0, q=FAKE, qd=sv.SV_BF16, pos0=FAKE):
        n = ctypes.c_size_t(0)
        return lib.spec_verify_sample(ctypes.byref(m), sv.SV_IN_HIDDEN, FAKE, 2, 4, FAKE, q, qd, T, 7, pos0, None,
                                      FAKE, FAKE, None, None, None, ctypes.byref(n), None)

    assert sample() == 0
    assert sample(T=-1.0) == 1
    assert sample(T=float("nan")) == 1
    assert sample(T=float("inf")) == 1
    assert sample(q=None) == 1
    assert sample(pos0=None) == 1
    assert sample(qd=5) == 2
    assert sample(T=0.0, q=None, pos0=None) == 0          # T == 0 is the greedy rule


def test_workspace_query_and_size_check(lib):
    m = _model(vocab=262144, d=1536)
    st, need = greedy(lib, m)
    assert st == 0 and need > 262144 * 5 * 4                # holds the float32 logits
    st, need_b8 = greedy(lib, m, B=8)
    assert st == 0 and need_b8 > need
    # too small / misaligned workspace: rejected on the host
    assert greedy(lib, m, ws=FAKE, nbytes=need - 1)[0] == 4
    assert greedy(lib, m, ws=ctypes.c_void_p(0x20008), nbytes=need)[0] == 4
    # logits input needs no logits buffer
    st, need_l = greedy(lib, sv.logits_model(262144).struct, kind=sv.SV_IN_LOGITS)
    assert st == 0 and need_l < need


def test_timing_api(lib):
    assert lib.sv_timing_enable(7) == 0
    ms, cnt = ctypes.c_double(1.0), ctypes.c_int64(5)
    assert lib.sv_timing_read(0, ctypes.byref(ms), ctypes.byref(cnt)) == 0
    assert cnt.value == 0 and ms.value == 0.0
    assert lib.sv_timing_enable(0) == 0


def test_masked_head_argument_errors_and_query(lib):
    def call(V=262144, d=1536, C=2048, wd=sv.SV_BF16, M=1, k=32, hidden=FAKE, clusters=FAKE, cl=None, ws=None,
             nbytes=0):
        h = sv._SvMaskedHead()
        h.vocab, h.d_model, h.n_clusters, h.wdtype = V, d, C, wd
        h.embed, h.centroids = 0x10000, 0x30000
        n = ctypes.c_size_t(nbytes)
        st = lib.draft_masked_logits(ctypes.byref(h), hidden, M, k, clusters, FAKE, cl, ws, ctypes.byref(n), None)
        return st, n.value

    st, need = call()
    assert st == 0 and need >= 2048 * 4                 # the cluster scores live in the workspace
    st, small = call(cl=FAKE)                            # caller keeps them: only the counter block
    assert st == 0 and 0 < small < need                  # never 0: a NULL ws is always the size query
    assert call(hidden=None)[0] == 1
    assert call(clusters=None)[0] == 1
    assert call(wd=sv.SV_F32)[0] == 2
    assert call(V=262145)[0] == 3                        # not a multiple of the cluster count
    assert call(C=8192, V=8192 * 4)[0] == 6             # more clusters than the selection sorts
    assert call(d=48)[0] == 3
    assert call(M=0)[0] == 1 and call(M=25)[0] == 1
    assert call(k=0)[0] == 1 and call(k=2049)[0] == 1
    assert call(ws=FAKE, nbytes=need - 1)[0] == 4


def test_filtered_sampling_argument_errors_and_query(lib):
    m = _model(vocab=262144, d=1536)

    def call(T=1.0, k=64, p=0.95, q=FAKE, pos0=FAKE, V=None, ws=None, nbytes=0):
        mm = _model(vocab=V, d=1536) if V else m
        n = ctypes.c_size_t(nbytes)
        st = lib.spec_verify_sample_filtered(ctypes.byref(mm), sv.SV_IN_HIDDEN, FAKE, 2, 4, FAKE, q, sv.SV_BF16, T,
                                             k, p, 7, pos0, None, FAKE, FAKE, None, ws, ctypes.byref(n), None)
        return st, n.value

    st, need = call()
    st_plain, need_plain = greedy(lib, m, B=2)
    assert st == 0 and st_plain == 0 and need > need_plain   # plus the candidate and kept lists
    assert call(T=-1.0)[0] == 1 and call(T=float("nan"))[0] == 1
    assert call(k=0)[0] == 6 and call(k=65)[0] == 6
    assert call(p=0.0)[0] == 1 and call(p=1.5)[0] == 1 and call(p=float("nan"))[0] == 1
    assert call(q=None)[0] == 1 and call(pos0=None)[0] == 1
    assert call(V=262144 + 4096)[0] == 6                       # 65 chunks x 64 candidates
    assert call(V=262144 + 4096, k=32)[0] == 0
    assert call(T=0.0, q=None, pos0=None)[0] == 0             # T == 0 is the greedy rule
    assert call(ws=FAKE, nbytes=need - 1)[0] == 4


def test_drafter_argument_errors_and_query(lib):
    ptrs = (ctypes.c_void_p * 28)(*([0x40000] * 28))
    kvp = (ctypes.c_void_p * 4)(*([0x50000] * 4))

    def call(nl=4, D=1536, H=256, nh=4, hd=128, ff=2048, V=262144, C=2048, tk=32, cent=True, B=1, gamma=4, T=1.0,
             q=FAKE, qd=sv.SV_F32, max_len=2048, ws=None, nbytes=0):
        d = sv._SvDrafter()
        d.n_layers, d.d_model, d.hidden, d.n_heads, d.head_dim, d.d_ff, d.vocab = nl, D, H, nh, hd, ff, V
        d.rms_eps, d.rope_theta = 1e-5, 10000.0
        d.embed = d.pre_proj = d.final_norm = d.post_proj = 0x10000
        d.layers = ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p))
        d.centroids = 0x30000 if cent else None
        d.n_clusters, d.top_k_clusters = C, tk
        k = sv._SvSharedKV()
        k.k = k.v = ctypes.cast(kvp, ctypes.POINTER(ctypes.c_void_p))
        k.max_len, k.len = max_len, 0x60000
        n = ctypes.c_size_t(nbytes)
        st = lib.mtp_draft(ctypes.byref(d), ctypes.byref(k), B, gamma, FAKE, FAKE, T, 5, FAKE, q, qd, ws,
                           ctypes.byref(n), None)
        return st, n.value

    st, need = call()
    assert st == 0 and need >= 32 * 128 * 4               # the scored logits live in the workspace
    st, need_tied = call(cent=False)
    assert st == 0 and need_tied >= 262144 * 4           # every token scored
    assert call(T=0.0, q=None)[0] == 0                   # greedy drafting needs no q
    assert call(q=None)[0] == 1 and call(T=-1.0)[0] == 1 and call(qd=7)[0] == 2
    assert call(nl=0)[0] == 1 and call(gamma=0)[0] == 1 and call(gamma=16)[0] == 1
    assert call(D=48)[0] == 3 and call(H=40)[0] == 3 and call(hd=96)[0] == 3 and call(ff=50)[0] == 3
    assert call(V=262145)[0] == 3                        # not a multiple of the cluster count
    assert call(C=8192, V=8192 * 32)[0] == 6 and call(tk=65)[0] == 1
    assert call(B=25)[0] == 1 and call(B=25, cent=False)[0] == 0
    assert call(max_len=0)[0] == 1
    assert call(ws=FAKE, nbytes=need - 1)[0] == 4


def test_round_policy_argument_errors(lib):
    n = ctypes.c_size_t(0)
    assert lib.round_pad_drafts(0, 4, 10, FAKE, FAKE, None, sv.SV_F32, 0.0, None, ctypes.byref(n), None) == 1
    assert lib.round_pad_drafts(2, 16, 10, FAKE, FAKE, None, sv.SV_F32, 0.0, None, ctypes.byref(n), None) == 1
    assert lib.round_pad_drafts(2, 4, 10, None, FAKE, None, sv.SV_F32, 0.0, None, ctypes.byref(n), None) == 1
    assert lib.round_pad_drafts(2, 4, 10, FAKE, FAKE, None, sv.SV_F32, 0.5, None, ctypes.byref(n), None) == 1
    assert lib.round_pad_drafts(2, 4, 10, FAKE, FAKE, FAKE, 9, 0.0, None, ctypes.byref(n), None) == 2
    assert lib.round_pad_drafts(2, 4, 10, FAKE, FAKE, FAKE, sv.SV_F32, 0.5, None, ctypes.byref(n), None) == 0
    assert n.value >= 2 * 4 * 4                          # the per-step confidences
    assert lib.round_update_gamma(2, FAKE, FAKE, 0, 4, None) == 1
    assert lib.round_update_gamma(2, FAKE, FAKE, 5, 4, None) == 1
    assert lib.round_update_gamma(2, None, FAKE, 1, 4, None) == 1
    assert lib.round_select_candidates(2, 3, 1, FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert lib.round_select_candidates(2, 0, 5, FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert lib.round_select_candidates(2, 3, 5, FAKE, None, None, FAKE, FAKE, None) == 1


def test_options(lib):
    """sv_set_option: the wait limit is accepted (and restored), an unknown option is an
    argument error with a message; no device is touched."""
    assert lib.sv_set_option(sv.SV_OPT_WAIT_LIMIT, 0) == 0
    assert lib.sv_set_option(sv.SV_OPT_WAIT_LIMIT, -1) == 0
    assert lib.sv_set_option(12345, 1) == 1
    assert b"unknown option" in lib.sv_last_error()


def test_noalloc_refuses_oversized_request_without_device(lib):
    """The allocation-free entry point checks its scratch size on the host, before any
    device call: a request whose scratch exceeds the fixed array is SV_ERR_UNSUPPORTED."""
    m = _model(vocab=65536, d=256)
    st = lib.spec_verify_sample_noalloc(ctypes.byref(m), sv.SV_IN_HIDDEN, FAKE, 64, 8, FAKE, FAKE, sv.SV_BF16,
                                        ctypes.c_float(1.0), ctypes.c_uint64(1), FAKE, None, FAKE, FAKE, None, None,
                                        None)
    assert st == 6 and b"scratch" in lib.sv_last_error()
    # argument errors come first, as on the workspace entry point
    st = lib.spec_verify_sample_noalloc(ctypes.byref(m), sv.SV_IN_HIDDEN, FAKE, 1, 0, FAKE, FAKE, sv.SV_BF16,
                                        ctypes.c_float(1.0), ctypes.c_uint64(1), FAKE, None, FAKE, FAKE, None, None,
                                        None)
    assert st == 1


def test_diag_is_optional_and_sized(lib):
    """diag = NULL computes nothing and needs no extra scratch; a non-NULL diag plans its
    partials (and the logits buffer) in the workspace query."""
    m = _model(vocab=262144, d=1536)
    st, need = greedy(lib, m)
    st2, need_diag = greedy(lib, m, diag=FAKE)
    assert st == 0 and st2 == 0 and need_diag > need


def test_tuning_entry_points_without_device(lib):
    """sv_tune_verify checks its arguments before touching a device; models it does not
    tune are left alone; sv_tuned_item reports nothing tuned."""
    h = sv._SvModel()
    h.n_layers, h.vocab, h.d_model, h.wdtype, h.lm_head = 0, 262144, 1536, sv.SV_BF16, FAKE
    assert lib.sv_tune_verify(None, 1, 4, None) == 1
    h32 = sv._SvModel()
    h32.n_layers, h32.vocab, h32.d_model, h32.wdtype, h32.lm_head = 0, 1024, 64, sv.SV_F32, FAKE
    assert lib.sv_tune_verify(ctypes.byref(h32), 1, 4, None) == 0          # float32 heads: nothing to tune
    assert lib.sv_tune_verify(ctypes.byref(h), 0, 4, None) == 1            # B out of range
    assert lib.sv_tune_verify(ctypes.byref(h), 1, 0, None) == 1            # gamma out of range
    assert lib.sv_tuned_item(ctypes.byref(h), 1, 4) == 0
