"""CPU checks of the C ABI: the library loads without a GPU, exports every
function include/dflash2.h declares, and rejects bad arguments with the
documented status before anything is launched.  Every call here has at
least one invalid argument, so nothing reaches the GPU runtime."""
import ctypes as C
import os
import re

import pytest

import draft_selection_bf16_amd as df2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = C.c_void_p(0x100000)      # aligned non-null stand-in; never dereferenced here


def _declared():
    src = open(os.path.join(ROOT, "include", "dflash2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash2_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = df2.lib()
    declared = _declared()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(df2.EXPORTS)


def test_version_and_strings():
    assert df2.dflash2_abi_version() == 2
    assert df2.dflash2_status_string(0) == "ok"
    assert df2.dflash2_status_string(4) == "workspace too small"


def _last():
    return df2.lib().dflash2_last_error().decode()


def test_topk_validation():
    L = df2.lib()
    assert L.dflash2_topk(FAKE, 7, 4, 1000, 16, FAKE, FAKE, FAKE, 1 << 20, None) == df2.DF2_ERR_DTYPE
    assert "dense" in _last()
    assert L.dflash2_topk(FAKE, 1, 4, 1000, 17, FAKE, FAKE, FAKE, 1 << 20, None) == df2.DF2_ERR_SHAPE
    assert L.dflash2_topk(FAKE, 1, 4, 10, 16, FAKE, FAKE, FAKE, 1 << 20, None) == df2.DF2_ERR_SHAPE
    assert L.dflash2_topk(FAKE, 1, 4, 1000, 0, FAKE, FAKE, FAKE, 1 << 20, None) == df2.DF2_ERR_SHAPE
    assert L.dflash2_topk(None, 1, 4, 1000, 16, FAKE, FAKE, FAKE, 1 << 20, None) == df2.DF2_ERR_NULL
    # few rows: the rows are split into chunks whose partial lists need workspace
    need = df2.dflash2_topk_workspace_bytes(15, 151936, 16)
    assert need > 0
    assert L.dflash2_topk(FAKE, 1, 15, 151936, 16, FAKE, FAKE, FAKE, need - 1, None) == \
        df2.DF2_ERR_WORKSPACE
    # zero rows is a no-op and succeeds without touching the runtime
    assert L.dflash2_topk(None, 1, 0, 1000, 16, None, None, None, 0, None) == df2.DF2_OK


def test_lm_head_topk_validation():
    L = df2.lib()
    need = df2.dflash2_lm_head_topk_workspace_bytes(480, 151936, 5120, 16)
    assert need >= 480 * 16 * 8
    f = L.dflash2_lm_head_topk
    a = lambda **kw: [kw.get("h", FAKE), FAKE, kw.get("dt", 1), kw.get("V", 151936), kw.get("rows", 480),
                      kw.get("d", 5120), kw.get("k", 16), FAKE, FAKE, FAKE, kw.get("ws", need), None]
    assert f(*a(dt=2)) == df2.DF2_ERR_DTYPE
    assert f(*a(d=100)) == df2.DF2_ERR_SHAPE
    assert f(*a(k=17)) == df2.DF2_ERR_SHAPE
    assert f(*a(k=0)) == df2.DF2_ERR_SHAPE
    assert f(*a(V=8)) == df2.DF2_ERR_SHAPE          # k > vocab
    assert f(*a(h=None)) == df2.DF2_ERR_NULL
    assert f(*a(h=C.c_void_p(0x100008))) == df2.DF2_ERR_SHAPE
    assert f(*a(ws=need - 1)) == df2.DF2_ERR_WORKSPACE
    assert f(None, None, 1, 151936, 0, 5120, 16, None, None, None, 0, None) == df2.DF2_OK


def test_verify_greedy_head_validation():
    L = df2.lib()
    need = df2.dflash2_verify_greedy_head_workspace_bytes(32, 15, 151936, 5120)
    assert need >= 32 * 16 * 8
    f = L.dflash2_verify_greedy_head
    a = lambda **kw: [kw.get("h", FAKE), FAKE, kw.get("dt", 1), 151936, kw.get("d", 5120), FAKE, kw.get("B", 32),
                      kw.get("T", 15), FAKE, FAKE, FAKE, kw.get("ws", need), None]
    assert f(*a(dt=0)) == df2.DF2_ERR_DTYPE
    assert f(*a(d=96)) == df2.DF2_ERR_SHAPE
    assert f(*a(T=64)) == df2.DF2_ERR_SHAPE
    assert f(*a(h=None)) == df2.DF2_ERR_NULL
    assert f(*a(ws=need - 1)) == df2.DF2_ERR_WORKSPACE
    assert f(None, None, 1, 151936, 5120, None, 0, 15, None, None, None, 0, None) == df2.DF2_OK


def test_verify_reject_head_validation():
    L = df2.lib()
    need = df2.dflash2_verify_reject_head_workspace_bytes(32, 15, 151936, 5120, 16)
    # block partials of every row and 128-token block dominate the workspace
    assert need >= 32 * 16 * ((151936 + 127) // 128) * 16
    f = L.dflash2_verify_reject_head
    a = lambda **kw: [kw.get("h", FAKE), FAKE, kw.get("dt", 1), 151936, kw.get("d", 5120), FAKE, FAKE, FAKE,
                      FAKE, kw.get("B", 32), kw.get("T", 15), kw.get("K", 16), kw.get("tau", 1.0), FAKE,
                      kw.get("b0", 0), FAKE, FAKE, FAKE, kw.get("ws", need), None]
    assert f(*a(dt=0)) == df2.DF2_ERR_DTYPE
    assert f(*a(tau=0.0)) == df2.DF2_ERR_UNSUPPORTED
    assert f(*a(tau=float("inf"))) == df2.DF2_ERR_UNSUPPORTED
    assert f(*a(d=96)) == df2.DF2_ERR_SHAPE
    assert f(*a(T=64)) == df2.DF2_ERR_SHAPE
    assert f(*a(K=17)) == df2.DF2_ERR_SHAPE
    assert f(*a(B=16385)) == df2.DF2_ERR_SHAPE
    assert f(*a(b0=-1)) == df2.DF2_ERR_SHAPE
    assert f(*a(b0=2 ** 31 - 32)) == df2.DF2_ERR_SHAPE
    assert f(*a(h=None)) == df2.DF2_ERR_NULL
    assert f(*a(ws=need - 1)) == df2.DF2_ERR_WORKSPACE
    assert f(None, None, 1, 151936, 5120, None, None, None, None, 0, 15, 16, 1.0, None, 0, None, None, None, 0,
             None) == df2.DF2_OK


def test_cycle_fused_validation():
    L = df2.lib()
    need = df2.dflash2_cycle_fused_workspace_bytes(1, 7, 16, 151936, 5120, 256)
    assert need > 0
    f = L.dflash2_cycle_fused
    a = lambda **kw: [FAKE, kw.get("ldt", 1), FAKE, kw.get("tdt", 1), 151936, FAKE, 1, kw.get("h", FAKE), FAKE,
                      FAKE, FAKE, FAKE, kw.get("B", 1), kw.get("T", 7), kw.get("K", 16), kw.get("d", 5120),
                      kw.get("r", 256), kw.get("gate", 0), kw.get("mode", 0)] + [FAKE] * 10 + [FAKE, kw.get("ws", need),
                                                                                      None]
    assert f(*a(ldt=0)) == df2.DF2_ERR_DTYPE
    assert f(*a(tdt=2)) == df2.DF2_ERR_DTYPE
    assert f(*a(mode=2)) == df2.DF2_ERR_UNSUPPORTED      # SAMPLE paths run in the multi-launch cycle
    assert f(*a(gate=3)) == df2.DF2_ERR_UNSUPPORTED
    assert f(*a(T=64)) == df2.DF2_ERR_SHAPE
    assert f(*a(B=147)) == df2.DF2_ERR_SHAPE               # B T > 1024
    assert f(*a(K=17)) == df2.DF2_ERR_SHAPE
    assert f(*a(d=100)) == df2.DF2_ERR_SHAPE
    assert f(*a(r=8)) == df2.DF2_ERR_SHAPE
    assert f(*a(h=None)) == df2.DF2_ERR_NULL
    assert f(*a(ws=need - 1)) == df2.DF2_ERR_WORKSPACE
    assert f(*a(B=0)) == df2.DF2_OK
    g = L.dflash2_cycle_fused_init
    assert g(1, 7, 16, 151936, 5120, 256, FAKE, need - 1, None) == df2.DF2_ERR_WORKSPACE
    assert g(1, 64, 16, 151936, 5120, 256, FAKE, need, None) == df2.DF2_ERR_SHAPE


def test_pair_scores_validation():
    L = df2.lib()
    args = lambda **kw: [kw.get("ci", FAKE), FAKE, FAKE, FAKE, kw.get("edt", 1), 151936, FAKE, FAKE,
                         FAKE, FAKE, kw.get("B", 2), kw.get("T", 7), kw.get("K", 16),
                         kw.get("d", 5120), kw.get("r", 256), kw.get("gate", 0), FAKE, FAKE,
                         kw.get("ws", 1 << 30), None]
    assert L.dflash2_pair_scores(*args(edt=0)) == df2.DF2_ERR_DTYPE
    assert L.dflash2_pair_scores(*args(d=100)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores(*args(r=8)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores(*args(r=264)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores(*args(K=17)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores(*args(T=0)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores(*args(T=64)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores(*args(gate=5)) == df2.DF2_ERR_UNSUPPORTED
    assert L.dflash2_pair_scores(*args(ci=None)) == df2.DF2_ERR_NULL
    need = df2.dflash2_pair_scores_workspace_bytes(2, 7, 16, 5120, 256)
    assert L.dflash2_pair_scores(*args(ws=need - 1)) == df2.DF2_ERR_WORKSPACE


def test_selector_tables_validation():
    L = df2.lib()
    args = lambda **kw: [kw.get("emb", FAKE), kw.get("edt", 1), kw.get("V", 151936), kw.get("d", 5120), FAKE,
                         FAKE, kw.get("r", 256), kw.get("tab", FAKE), None]
    assert L.dflash2_selector_tables(*args(edt=0)) == df2.DF2_ERR_DTYPE
    assert L.dflash2_selector_tables(*args(d=100)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_selector_tables(*args(r=8)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_selector_tables(*args(r=272)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_selector_tables(*args(V=-1)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_selector_tables(*args(V=1 << 20, d=4096)) == df2.DF2_ERR_UNSUPPORTED
    assert L.dflash2_selector_tables(*args(tab=None)) == df2.DF2_ERR_NULL
    assert L.dflash2_selector_tables(*args(tab=C.c_void_p(0x100004))) == df2.DF2_ERR_SHAPE
    assert L.dflash2_selector_tables(None, 1, 0, 5120, None, None, 256, None, None) == df2.DF2_OK


def test_pair_scores_tab_validation():
    L = df2.lib()
    need = df2.dflash2_pair_scores_tab_workspace_bytes(32, 16, 5120, 256)
    assert need > 0
    assert need < df2.dflash2_pair_scores_workspace_bytes(32, 16, 16, 5120, 256)
    args = lambda **kw: [kw.get("ci", FAKE), FAKE, FAKE, kw.get("tab", FAKE), 151936, FAKE, FAKE,
                         kw.get("B", 32), kw.get("T", 16), kw.get("K", 16), kw.get("d", 5120),
                         kw.get("r", 256), kw.get("gate", 0), FAKE, FAKE, kw.get("ws", need), None]
    assert L.dflash2_pair_scores_tab(*args(T=0)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores_tab(*args(T=64)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores_tab(*args(K=17)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores_tab(*args(d=96)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores_tab(*args(r=20)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores_tab(*args(gate=2)) == df2.DF2_ERR_UNSUPPORTED
    assert L.dflash2_pair_scores_tab(*args(tab=None)) == df2.DF2_ERR_NULL
    assert L.dflash2_pair_scores_tab(*args(tab=C.c_void_p(0x100008))) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores_tab(*args(ws=need - 1)) == df2.DF2_ERR_WORKSPACE


def test_h_projection_and_from_h_validation():
    L = df2.lib()
    need = df2.dflash2_pair_scores_tab_workspace_bytes(32, 16, 5120, 256)
    assert L.dflash2_h_projection(FAKE, FAKE, 32, 16, 100, 256, FAKE, need, None) == df2.DF2_ERR_SHAPE
    assert L.dflash2_h_projection(FAKE, FAKE, 32, 0, 5120, 256, FAKE, need, None) == df2.DF2_ERR_SHAPE
    assert L.dflash2_h_projection(None, FAKE, 32, 16, 5120, 256, FAKE, need, None) == df2.DF2_ERR_NULL
    assert L.dflash2_h_projection(FAKE, FAKE, 32, 16, 5120, 256, FAKE, need - 1, None) == df2.DF2_ERR_WORKSPACE
    assert L.dflash2_h_projection(None, None, 0, 16, 5120, 256, None, 0, None) == df2.DF2_OK
    args = lambda **kw: [FAKE, FAKE, FAKE, kw.get("tab", FAKE), 151936, 32, 16, kw.get("K", 16), 5120, 256,
                         kw.get("gate", 0), FAKE, FAKE, kw.get("ws", need), None]
    assert L.dflash2_pair_scores_tab_from_h(*args(K=0)) == df2.DF2_ERR_SHAPE
    assert L.dflash2_pair_scores_tab_from_h(*args(gate=3)) == df2.DF2_ERR_UNSUPPORTED
    assert L.dflash2_pair_scores_tab_from_h(*args(tab=None)) == df2.DF2_ERR_NULL
    assert L.dflash2_pair_scores_tab_from_h(*args(ws=need - 1)) == df2.DF2_ERR_WORKSPACE


def test_path_validation():
    L = df2.lib()
    f = L.dflash2_path_viterbi
    assert f(FAKE, FAKE, 2, 7, 16, 3, 1.0, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None) == df2.DF2_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, 2, 7, 16, 2, 0.0, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None) == df2.DF2_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, 2, 7, 16, 2, float("inf"), FAKE, 0, FAKE, FAKE, FAKE, FAKE, None) == \
        df2.DF2_ERR_UNSUPPORTED
    assert f(FAKE, FAKE, 2, 7, 16, 2, 1.0, None, 0, FAKE, FAKE, FAKE, FAKE, None) == df2.DF2_ERR_NULL
    assert f(FAKE, FAKE, 2, 7, 0, 0, 1.0, None, 0, FAKE, FAKE, FAKE, FAKE, None) == df2.DF2_ERR_SHAPE
    assert f(None, FAKE, 2, 7, 16, 0, 0.0, None, 0, FAKE, FAKE, FAKE, FAKE, None) == df2.DF2_ERR_NULL
    # the request offset of the Philox counters: b0 >= 0 and b0 + B < 2^31
    assert f(FAKE, FAKE, 2, 7, 16, 2, 1.0, FAKE, -1, FAKE, FAKE, FAKE, FAKE, None) == df2.DF2_ERR_SHAPE
    assert f(FAKE, FAKE, 2, 7, 16, 2, 1.0, FAKE, 2**31 - 2, FAKE, FAKE, FAKE, FAKE, None) == df2.DF2_ERR_SHAPE


def test_conv_validation():
    L = df2.lib()
    need = df2.dflash2_dynconv2_workspace_bytes(32, 16, 5120)
    assert need > 0
    assert L.dflash2_dynconv2(FAKE, FAKE, FAKE, None, 32, 16, 5120, 16, FAKE, 2, FAKE, need, None) == \
        df2.DF2_ERR_DTYPE
    assert L.dflash2_dynconv2(FAKE, FAKE, FAKE, None, 32, 16, 5120, 8, FAKE, 1, FAKE, need, None) == \
        df2.DF2_ERR_SHAPE
    assert L.dflash2_dynconv2(FAKE, FAKE, FAKE, None, 32, 16, 5000, 16, FAKE, 1, FAKE, need, None) == \
        df2.DF2_ERR_SHAPE
    assert L.dflash2_dynconv2(FAKE, FAKE, FAKE, None, 32, 0, 5120, 16, FAKE, 1, FAKE, need, None) == \
        df2.DF2_ERR_SHAPE
    assert L.dflash2_dynconv2(None, FAKE, FAKE, None, 32, 16, 5120, 16, FAKE, 1, FAKE, need, None) == \
        df2.DF2_ERR_NULL
    assert L.dflash2_dynconv2(C.c_void_p(0x100002), FAKE, FAKE, None, 32, 16, 5120, 16, FAKE, 1, FAKE,
                              need, None) == df2.DF2_ERR_SHAPE
    assert L.dflash2_dynconv2(FAKE, FAKE, FAKE, None, 32, 16, 5120, 16, FAKE, 1, FAKE, need - 1,
                              None) == df2.DF2_ERR_WORKSPACE


def test_verify_validation():
    L = df2.lib()
    need = df2.dflash2_verify_workspace_bytes(32, 15, 151936)
    assert need > 0
    assert L.dflash2_verify_greedy(FAKE, 5, 151936, FAKE, 32, 15, FAKE, FAKE, FAKE, need, None) == \
        df2.DF2_ERR_DTYPE
    assert L.dflash2_verify_greedy(FAKE, 1, 151936, FAKE, 32, 64, FAKE, FAKE, FAKE, need, None) == \
        df2.DF2_ERR_SHAPE
    assert L.dflash2_verify_greedy(FAKE, 1, 151936, None, 32, 15, FAKE, FAKE, FAKE, need, None) == \
        df2.DF2_ERR_NULL
    assert L.dflash2_verify_greedy(FAKE, 1, 151936, FAKE, 32, 15, FAKE, FAKE, FAKE, need - 1, None) == \
        df2.DF2_ERR_WORKSPACE
    args = [FAKE, 1, 151936, FAKE, FAKE, FAKE, FAKE, 32, 15, 16]
    tail = [FAKE, 0, FAKE, FAKE, FAKE, need, None]
    assert L.dflash2_verify_reject(*args, 0.0, *tail) == df2.DF2_ERR_UNSUPPORTED
    assert L.dflash2_verify_reject(*args, -1.0, *tail) == df2.DF2_ERR_UNSUPPORTED
    assert L.dflash2_verify_reject(*args, 1.0, None, *tail[1:]) == df2.DF2_ERR_NULL
    assert L.dflash2_verify_reject(*args[:-1], 0, 1.0, *tail) == df2.DF2_ERR_SHAPE
    assert L.dflash2_verify_reject(*args, 1.0, *tail[:-2], need - 1, None) == df2.DF2_ERR_WORKSPACE
    assert L.dflash2_verify_reject(*args, 1.0, FAKE, -3, *tail[2:]) == df2.DF2_ERR_SHAPE
    assert L.dflash2_verify_reject(*args, 1.0, FAKE, 2**31 - 32, *tail[2:]) == df2.DF2_ERR_SHAPE


def test_verify_greedy_noalloc_validation():
    """The allocation-free greedy verification checks its arguments, and
    rejects a size whose scratch exceeds its fixed array, before it looks up
    the array or launches anything."""
    L = df2.lib()
    f = L.dflash2_verify_greedy_noalloc
    assert df2.dflash2_verify_greedy_noalloc_max_bytes() == 1 << 20
    assert f(FAKE, 5, 151936, FAKE, 32, 15, FAKE, FAKE, None) == df2.DF2_ERR_DTYPE
    assert f(FAKE, 1, 151936, FAKE, 32, 64, FAKE, FAKE, None) == df2.DF2_ERR_SHAPE
    assert f(FAKE, 1, 151936, None, 32, 15, FAKE, FAKE, None) == df2.DF2_ERR_NULL
    assert f(C.c_void_p(0x100001), 1, 151936, FAKE, 32, 15, FAKE, FAKE, None) == df2.DF2_ERR_SHAPE
    assert df2.dflash2_verify_workspace_bytes(4096, 15, 151936) > (1 << 20)
    assert f(FAKE, 1, 151936, FAKE, 4096, 15, FAKE, FAKE, None) == df2.DF2_ERR_WORKSPACE
    assert "scratch" in _last()
    assert f(None, 1, 151936, None, 0, 15, None, None, None) == df2.DF2_OK


def test_empty_batch_is_a_no_op():
    """A batch of zero requests is valid everywhere: each entry point checks
    its sizes and returns DF2_OK before it touches a pointer or the runtime
    (all data pointers here are NULL)."""
    L = df2.lib()
    assert L.dflash2_topk(None, 1, 0, 151936, 16, None, None, None, 0, None) == df2.DF2_OK
    assert L.dflash2_pair_scores(None, None, None, None, 1, 151936, None, None, None, None, 0, 7, 16, 5120,
                                 256, 0, None, None, 0, None) == df2.DF2_OK
    for mode in (0, 1, 2):
        assert L.dflash2_path_viterbi(None, None, 0, 7, 16, mode, 1.0, None, 0, None, None, None, None,
                                      None) == df2.DF2_OK
    assert L.dflash2_pair_scores_tab(None, None, None, None, 151936, None, None, 0, 7, 16, 5120, 256, 0, None,
                                     None, 0, None) == df2.DF2_OK
    assert L.dflash2_dynconv2(None, None, None, None, 0, 16, 5120, 16, None, 1, None, 0, None) == df2.DF2_OK
    assert L.dflash2_verify_greedy(None, 1, 151936, None, 0, 15, None, None, None, 0, None) == df2.DF2_OK
    assert L.dflash2_verify_reject(None, 1, 151936, None, None, None, None, 0, 15, 16, 1.0, None, 0, None,
                                   None, None, 0, None) == df2.DF2_OK


def test_philox_validation():
    L = df2.lib()
    assert L.dflash2_philox4x64(FAKE, FAKE, FAKE, -1, FAKE, None) == df2.DF2_ERR_SHAPE
    assert L.dflash2_philox4x64(None, FAKE, FAKE, 4, FAKE, None) == df2.DF2_ERR_NULL
    assert L.dflash2_philox4x64(None, None, None, 0, None, None) == df2.DF2_OK


def test_binding_raises_on_error():
    import torch
    x = torch.zeros(4, 10, dtype=torch.float64)     # unsupported dtype
    with pytest.raises(df2.DFlash2Error) as e:
        df2.dflash2_topk(x, 4, x, x, None, stream=type("S", (), {"cuda_stream": 0})())
    assert e.value.status == df2.DF2_ERR_DTYPE
