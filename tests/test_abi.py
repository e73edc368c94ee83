"""The C-ABI library on the host: it loads, exports what include/occ.h
declares, and rejects bad arguments before any launch (so these run without
a GPU).  The host-side greedy placement is checked against the oracle."""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def occ():
    if not os.path.exists(os.path.join(ROOT, "expert_top_router_amd", "liboccult.so")):
        import __graft_entry__
        __graft_entry__._hip_build_module().build()
    import expert_top_router_amd as occ
    return occ


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "occ.h")).read()
    return set(re.findall(r"^(?:occ_status|size_t|const char \*)\s*(occ_\w+)\s*\(", src, re.M))


def test_every_declared_symbol_is_exported(occ):
    names = declared_symbols()
    assert len(names) == 29, names
    lib = C.CDLL(occ.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(occ.EXPORTED)


def _desc(occ, **kw):
    base = dict(T=64, d=64, E=8, k=2, D=2, I=128, n_shared=0, I_shared=0, dtype="bf16", renorm=0)
    base.update(kw)
    return occ.make_desc(**base)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("kw,code", [
    (dict(E=10, D=4), -1),          # E % D != 0
    (dict(k=9), -1),                # k > E
    (dict(T=-1), -1),
    (dict(dtype=7), -1),
    (dict(renorm=2), -1),
    (dict(E=256, D=2, k=2), -2),    # E beyond OCC_MAX_E
    (dict(E=64, D=64, k=17), -2),   # k beyond OCC_MAX_K
    (dict(E=128, D=64), -2),        # D beyond OCC_MAX_D
    (dict(d=60), -2),               # d % 8
    (dict(d=72), -2),               # bf16 GEMM tiles need d % 64
    (dict(I=96), -2),
    (dict(dtype="f32", d=4096), -2),  # 16 KiB rows
    (dict(n_shared=1, I_shared=0), -1),
])
def test_bad_descriptors_are_rejected(occ, kw, code):
    d = _desc(occ, **kw)
    rc = occ.lib().occ_route_topk(C.byref(d), FAKE, FAKE, FAKE, FAKE, None, None)
    assert rc == code, occ.last_error()
    assert occ.last_error()
    assert occ.occ_workspace_bytes(d) == 0



def test_route_workspace_only_on_the_filtered_path(occ):
    """occ_route_workspace_bytes is positive exactly where the candidate
    filter applies (bf16, 32 <= E <= 128, k <= 16, d % 64 == 0), and
    occ_route_topk_ws checks the workspace before it launches anything."""
    lib = occ.lib()
    on = _desc(occ, T=300, d=192, E=64, k=6, D=8)
    assert occ.occ_route_workspace_bytes(on) >= 300 * 64 * 4 + 64 * 192 * 2
    for kw in (dict(dtype="f32"), dict(E=16, D=2), dict(E=64, D=8, k=17), dict(d=200)):
        assert occ.occ_route_workspace_bytes(_desc(occ, **{**dict(T=300, d=192, E=64, k=6, D=8),
                                                           **kw})) == 0, kw
    n = occ.occ_route_workspace_bytes(on)
    assert lib.occ_route_topk_ws(C.byref(on), FAKE, FAKE, FAKE, FAKE, None, n, None) == -1
    assert lib.occ_route_topk_ws(C.byref(on), FAKE, FAKE, FAKE, FAKE, FAKE, n - 1, None) == -3
    assert "workspace" in occ.last_error()
    assert lib.occ_route_topk_ws(C.byref(on), None, FAKE, FAKE, FAKE, FAKE, n, None) == -1

def test_null_pointers_and_workspace(occ):
    d = _desc(occ)
    lib = occ.lib()
    assert lib.occ_route_topk(None, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert lib.occ_route_topk(C.byref(d), None, FAKE, FAKE, FAKE, None, None) == -1
    brim = occ.make_brim(brim0=FAKE, brim1=FAKE, sfd_offset=FAKE, slot_offset=FAKE,
                         sfd_token=FAKE, epd_token=FAKE, epd_sfd=FAKE, epd_w=FAKE, S=FAKE)
    se = np.arange(8, dtype=np.int32)
    need = occ.occ_workspace_bytes(d)
    assert need > 0
    rc = lib.occ_build_brim(C.byref(d), FAKE, FAKE, se.ctypes.data, C.byref(brim), FAKE,
                            need - 1, None)
    assert rc == -3 and "workspace" in occ.last_error()
    bad = np.array([0, 1, 2, 3, 4, 5, 6, 6], dtype=np.int32)
    rc = lib.occ_build_brim(C.byref(d), FAKE, FAKE, bad.ctypes.data, C.byref(brim), FAKE,
                            need, None)
    assert rc == -1 and "permutation" in occ.last_error()
    partial = occ.make_brim(brim0=FAKE, brim1=FAKE, slot_offset=FAKE)
    rc = lib.occ_build_brim(C.byref(d), FAKE, FAKE, se.ctypes.data, C.byref(partial), FAKE,
                            need, None)
    assert rc == -1


def test_noalloc_brim_arguments_are_checked(occ):
    """occ_build_brim_noalloc: occ_build_brim's checks, and layers whose
    workspace exceeds the library's fixed array are refused (no launch)."""
    lib = occ.lib()
    brim = occ.make_brim(brim0=FAKE, brim1=FAKE, sfd_offset=FAKE, slot_offset=FAKE,
                         sfd_token=FAKE, epd_token=FAKE, epd_sfd=FAKE, epd_w=FAKE, S=FAKE)
    se = np.arange(8, dtype=np.int32)
    d = _desc(occ)
    assert lib.occ_build_brim_noalloc(None, FAKE, FAKE, se.ctypes.data, C.byref(brim), None) == -1
    assert lib.occ_build_brim_noalloc(C.byref(d), None, FAKE, se.ctypes.data, C.byref(brim),
                                      None) == -1
    bad = np.array([0, 1, 2, 3, 4, 5, 6, 6], dtype=np.int32)
    assert lib.occ_build_brim_noalloc(C.byref(d), FAKE, FAKE, bad.ctypes.data, C.byref(brim),
                                      None) == -1
    partial = occ.make_brim(brim0=FAKE, brim1=FAKE, slot_offset=FAKE)
    assert lib.occ_build_brim_noalloc(C.byref(d), FAKE, FAKE, se.ctypes.data, C.byref(partial),
                                      None) == -1
    # 2^20 tokens with 16 devices and 128 experts: (16 + 128) keys x 16384
    # blocks of counts, far beyond the 1 MiB array
    big = _desc(occ, T=1 << 20, E=128, D=16, k=6)
    assert occ.occ_workspace_bytes(big) > 1 << 20
    se128 = np.arange(128, dtype=np.int32)
    rc = lib.occ_build_brim_noalloc(C.byref(big), FAKE, FAKE, se128.ctypes.data, C.byref(brim),
                                    None)
    assert rc == -2 and "occ_build_brim" in occ.last_error()
    # the largest workload of the suite (65536 tokens, 16 + 128 keys) fits
    c5 = _desc(occ, T=65536, d=2048, E=128, D=16, k=6, I=768)
    assert 0 < occ.occ_workspace_bytes(c5) <= 1 << 20


def test_pruned_brim_arguments_are_checked(occ):
    lib = occ.lib()
    d = _desc(occ)  # D = 2
    brim = occ.make_brim(brim0=FAKE, brim1=FAKE, sfd_offset=FAKE, slot_offset=FAKE,
                         sfd_token=FAKE, epd_token=FAKE, epd_sfd=FAKE, epd_w=FAKE, S=FAKE)
    se = np.arange(8, dtype=np.int32)
    need = occ.occ_workspace_bytes(d)
    for budget, rescale in [(0, 1), (3, 1), (-1, 0), (1, 2)]:
        rc = lib.occ_build_brim_pruned(C.byref(d), FAKE, FAKE, se.ctypes.data, budget, rescale,
                                       C.byref(brim), FAKE, need, None)
        assert rc == -1, (budget, rescale)
    rc = lib.occ_build_brim_pruned(C.byref(d), FAKE, FAKE, se.ctypes.data, 1, 1, C.byref(brim),
                                   FAKE, need - 1, None)
    assert rc == -3


def test_backward_arguments_are_checked(occ):
    lib = occ.lib()
    brim = occ.make_brim(brim0=FAKE, brim1=FAKE, sfd_offset=FAKE, slot_offset=FAKE,
                         sfd_token=FAKE, epd_token=FAKE, epd_sfd=FAKE, epd_w=FAKE, S=FAKE)
    se = np.arange(8, dtype=np.int32)
    d = _desc(occ)
    assert occ.occ_backward_workspace_bytes(d) == 2 * 64 * 2 * 2 * 128 * 2
    f32 = _desc(occ, dtype="f32")
    # fp32 layers: [G | U] and [dG | dU] in fp32
    assert occ.occ_backward_workspace_bytes(f32) == 2 * 64 * 2 * 2 * 128 * 4
    assert lib.occ_grad_combine(C.byref(f32), None, C.byref(brim), FAKE, None, FAKE, FAKE,
                                None) == -1
    sh = _desc(occ, n_shared=1, I_shared=64)
    # shared experts: grad-dispatch needs their input gradient, and only then
    assert lib.occ_grad_dispatch(C.byref(sh), FAKE, C.byref(brim), None, None, FAKE, FAKE,
                                 None) == -1
    assert lib.occ_grad_dispatch(C.byref(d), FAKE, C.byref(brim), None, FAKE, FAKE, FAKE,
                                 None) == -1
    assert lib.occ_grad_dispatch(C.byref(f32), FAKE, C.byref(brim), None, None, FAKE, None,
                                 None) == -1
    # occ_shared_backward: only for layers with shared experts; workspace checked
    hb_sh = occ.occ_ffn_workspace_bytes(sh)
    ws_sh = occ.occ_backward_workspace_bytes(sh)
    assert ws_sh >= 2 * 64 * 2 * 64 * 2
    assert lib.occ_shared_backward(C.byref(d), FAKE, FAKE, FAKE, FAKE, hb_sh, FAKE, FAKE, ws_sh,
                                   FAKE, FAKE, FAKE, None) == -1
    assert lib.occ_shared_backward(C.byref(sh), FAKE, FAKE, FAKE, FAKE, hb_sh, FAKE, FAKE,
                                   ws_sh, None, FAKE, FAKE, None) == -1
    assert lib.occ_shared_backward(C.byref(sh), FAKE, FAKE, FAKE, FAKE, hb_sh, FAKE, FAKE, 1,
                                   FAKE, FAKE, FAKE, None) == -3
    # the pair that keeps [G | U] stays without shared experts
    assert lib.occ_grad_combine(C.byref(d), None, C.byref(brim), FAKE, None, FAKE, FAKE,
                                None) == -1
    ws = occ.occ_backward_workspace_bytes(d)
    hb = occ.occ_ffn_workspace_bytes(d)
    rc = lib.occ_expert_backward(C.byref(d), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE,
                                 FAKE, hb, FAKE, FAKE, ws - 1, FAKE, FAKE, FAKE, None)
    assert rc == -3
    rc = lib.occ_expert_backward(C.byref(d), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE,
                                 FAKE, hb, FAKE, FAKE, ws, FAKE, None, FAKE, None)
    assert rc == -1
    rc = lib.occ_router_backward(C.byref(d), FAKE, FAKE, None, FAKE, FAKE, se.ctypes.data,
                                 C.byref(brim), FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert rc == -1
    # the pair that keeps [G | U]: bf16 without shared experts, gu required
    assert lib.occ_expert_ffn_keep(C.byref(f32), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE,
                                   FAKE, hb, FAKE, FAKE, None) == -2
    assert lib.occ_expert_ffn_keep(C.byref(sh), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE,
                                   FAKE, hb, FAKE, FAKE, None) == -2
    assert lib.occ_expert_ffn_keep(C.byref(d), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE,
                                   FAKE, hb, None, FAKE, None) == -1
    assert lib.occ_expert_ffn_keep(C.byref(d), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE,
                                   FAKE, hb - 1, FAKE, FAKE, None) == -3
    rc = lib.occ_expert_backward_kept(C.byref(d), FAKE, C.byref(brim), se.ctypes.data, FAKE,
                                      FAKE, FAKE, hb, None, FAKE, FAKE, ws, FAKE, FAKE, FAKE, None)
    assert rc == -1
    rc = lib.occ_expert_backward_kept(C.byref(d), FAKE, C.byref(brim), se.ctypes.data, FAKE,
                                      FAKE, FAKE, hb, FAKE, FAKE, FAKE, ws - 1, FAKE, FAKE, FAKE,
                                      None)
    assert rc == -3
    # [G | U] of T*k rows x 2I bf16 beyond 4 GiB (the backward GEMMs address
    # it with 32-bit offsets), although every forward operand fits
    wide = _desc(occ, T=65536, k=8, d=2048, E=64, D=8, I=3072)
    assert lib.occ_expert_ffn(C.byref(wide), None, None, None, None, None, None, 0, None, None,
                              None, None, None, None) == -1  # forward: passes the shape check
    assert occ.occ_backward_workspace_bytes(wide) == 0
    rc = lib.occ_expert_backward(C.byref(wide), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE,
                                 FAKE, hb, FAKE, FAKE, ws, FAKE, FAKE, FAKE, None)
    assert rc == -2
    assert lib.occ_grad_combine(C.byref(wide), FAKE, C.byref(brim), FAKE, None, FAKE, FAKE,
                                None) == -2
    # a long batch splits dW_r over token chunks, whose partial sums need the workspace
    big = _desc(occ, T=8192)
    rc = lib.occ_router_backward(C.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, se.ctypes.data,
                                 C.byref(brim), FAKE, FAKE, FAKE, FAKE, FAKE, 0, None)
    assert rc == -3


def test_affinity_arguments_are_checked(occ):
    lib = occ.lib()
    se = np.arange(8, dtype=np.int32)
    bad = np.array([0, 1, 2, 3, 4, 5, 6, 6], np.int32)
    assert lib.occ_cross_coactivation(10, 2, 8, FAKE, 9, 8, FAKE, FAKE, 0, None) == -1  # k > E
    assert lib.occ_cross_coactivation(10, 2, 8, None, 2, 8, FAKE, FAKE, 0, None) == -1
    assert lib.occ_cross_coactivation(10, 2, 256, FAKE, 2, 8, FAKE, FAKE, 0, None) == -2
    assert lib.occ_cross_coactivation(10, 2, 8, FAKE, 2, 8, FAKE, FAKE, 3, None) == -1
    assert lib.occ_home_device(10, 2, 8, FAKE, 8, 3, se.ctypes.data, FAKE, FAKE, None) == -1
    assert lib.occ_home_device(10, 2, 8, FAKE, 8, 2, bad.ctypes.data, FAKE, FAKE, None) == -1
    assert lib.occ_home_device(10, 2, 8, FAKE, 8, 2, se.ctypes.data, None, FAKE, None) == -1
    assert lib.occ_local_hits(10, 2, 8, FAKE, 2, se.ctypes.data, FAKE, None, 0, None) == -1
    assert lib.occ_local_hits(10, 2, 8, FAKE, 2, None, FAKE, FAKE, 0, None) == -1


def test_direct_mode_arguments_are_checked(occ):
    lib = occ.lib()
    d = _desc(occ)
    brim = occ.make_brim(brim0=FAKE, brim1=FAKE, slot_offset=FAKE, epd_w=FAKE)
    assert lib.occ_dispatch_direct(C.byref(d), None, C.byref(brim), FAKE, None) == -1
    assert lib.occ_dispatch_direct(C.byref(d), FAKE, C.byref(brim), None, None) == -1
    assert lib.occ_combine_direct(C.byref(d), None, C.byref(brim), None, FAKE, None) == -1
    assert lib.occ_combine_direct(C.byref(d), FAKE, C.byref(brim), None, None, None) == -1
    nw = occ.make_brim(brim0=FAKE, brim1=FAKE, slot_offset=FAKE)
    rc = lib.occ_combine_direct(C.byref(d), FAKE, C.byref(nw), None, FAKE, None)
    assert rc == -1 and "epd_w" in occ.last_error()
    bad = _desc(occ, E=10, D=4)
    assert lib.occ_dispatch_direct(C.byref(bad), FAKE, C.byref(brim), FAKE, None) == -1


def test_shared_expert_arguments_are_checked(occ):
    lib = occ.lib()
    brim = occ.make_brim(brim0=FAKE, brim1=FAKE, slot_offset=FAKE, epd_w=FAKE)
    se = np.arange(8, dtype=np.int32)
    d = _desc(occ, n_shared=2, I_shared=64)
    hb = occ.occ_ffn_workspace_bytes(d)
    assert hb == 64 * 2 * 128 * 2 + 64 * 2 * 64 * 2
    rc = lib.occ_expert_ffn(C.byref(d), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE, FAKE,
                            hb, FAKE, None, None, None, None, None)
    assert rc == -1 and "n_shared" in occ.last_error()
    d0 = _desc(occ)
    rc = lib.occ_expert_ffn(C.byref(d0), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE, FAKE,
                            occ.occ_ffn_workspace_bytes(d0), FAKE, FAKE, None, None, None, None)
    assert rc == -1
    rc = lib.occ_expert_ffn(C.byref(d0), FAKE, C.byref(brim), se.ctypes.data, FAKE, FAKE, FAKE,
                            10, FAKE, None, None, None, None, None)
    assert rc == -3


def test_greedy_placement_matches_oracle(occ, orc):
    rng = np.random.default_rng(0)
    for E, D in [(4, 2), (8, 2), (16, 4), (64, 8), (128, 16)]:
        for trial in range(5):
            k = min(6, E)
            idx = np.stack([rng.permutation(E)[:k] for _ in range(300)]).astype(np.int32)
            Cm = orc.coactivation(idx, E)
            if trial == 0:
                Cm = np.zeros((E, E), np.int32)  # all ties
            got = occ.occ_place_greedy(E, D, Cm)
            assert np.array_equal(got, orc.greedy_placement(Cm, D))
    with pytest.raises(occ.OccError):
        occ.occ_place_greedy(10, 4, np.zeros((10, 10), np.int32))
