"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/kvsel.h declares, answers workspace queries and rejects
bad arguments before any HIP call (nothing is launched on these paths)."""
import ctypes
import os
import re

import pytest

import eviction_importance_scoring_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvsel.h")

OK, ARG, UNSUP, WS = 0, 1, 2, 3

# Tests that pass made-up non-null pointers only ever hit argument checks;
# they are not run where a GPU is visible, so that a validation bug could
# never launch a kernel on a bogus address.
no_gpu_only = pytest.mark.skipif(
    __import__("torch").cuda.is_available(),
    reason="passes fake device pointers; CPU-only contract test")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kv.library_path):
        pytest.fail("libkvsel.so not built (run __graft_entry__.build())")
    return kv.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"kvsel_score", "kvsel_value_weight", "kvsel_select", "kvsel_compact",
                          "kvsel_status_str", "kvsel_abi_version"}
    for name in names:
        assert hasattr(lib, name), f"{name} declared in kvsel.h but not exported"


def test_select_static_checks(lib):
    """Checks run before any HIP call: a request needing more than the static
    scratch is refused with KVSEL_ERR_SCRATCH, missing pointers with ARG."""
    f = lib.kvsel_select_static
    assert lib.kvsel_static_scratch_bytes() == 16 << 20
    # 8000 segments of 50,000 candidates: the many-workgroup state alone is ~66 MB
    assert f(None, None, 1000, 8, 50000, 32, 1000, 0, 1.0, 1e-4, 0.5, None, None, None,
             None) == 5
    assert kv.kvsel_status_str(5).startswith("KVSEL_ERR_SCRATCH")
    assert f(None, None, 1, 8, 50000, 32, 1000, 0, 1.0, 1e-4, 0.5, None, None, None, None) == ARG
    assert f(None, None, 1, 8, 50000, 32, 20, 0, 1.0, 1e-4, 0.5, None, None, None, None) == ARG


def test_version_and_status_strings(lib):
    assert lib.kvsel_abi_version() == 2
    for code in (OK, ARG, UNSUP, WS, 4, 5):
        assert kv.kvsel_status_str(code).startswith("KVSEL")
    assert "unknown" in kv.kvsel_status_str(99)


def _score(lib, **kw):
    a = dict(L=1, H=8, G=4, d=128, n=4096, W=32, mode=0, agg=0, scale=0.088, pool=7)
    a.update(kw)
    nb = ctypes.c_size_t(0)
    rc = lib.kvsel_score(None, None, a["L"], a["H"], a["G"], a["d"], a["n"], a["W"], a["mode"],
                         a["agg"], a["scale"], a["pool"], None, None, None, ctypes.byref(nb), None)
    return rc, nb.value


def test_score_workspace_query(lib):
    rc, nb = _score(lib)
    assert rc == OK and nb > 0
    rc2, nb2 = _score(lib, L=32, n=32768)
    assert rc2 == OK and nb2 >= nb


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), ARG), (dict(H=0), ARG), (dict(G=0), ARG), (dict(n=0), ARG), (dict(W=0), ARG),
    (dict(W=4096), ARG), (dict(W=5000), ARG), (dict(mode=2), ARG), (dict(agg=3), ARG),
    (dict(scale=0.0), ARG), (dict(scale=-1.0), ARG), (dict(scale=float("inf")), ARG),
    (dict(scale=float("nan")), ARG), (dict(pool=0), ARG), (dict(pool=4), ARG),
    (dict(d=64), UNSUP), (dict(pool=67), UNSUP),
    # one head's K (or query rows) reaching 2^31 bytes: n * 256 >= 2^31
    (dict(H=1, n=1 << 23), UNSUP), (dict(H=1, G=1, n=1 << 23, W=(1 << 23) - 1), UNSUP),
    (dict(H=1, n=(1 << 23) - 1), OK), (dict(H=1, G=2, W=1 << 22, n=(1 << 22) + 1), UNSUP),
])
def test_score_rejects(lib, kw, code):
    assert _score(lib, **kw)[0] == code


def test_score_external_allows_w_ge_n(lib):
    assert _score(lib, mode=1, W=8192, n=4096)[0] == OK


@no_gpu_only
def test_score_null_and_workspace_checks(lib):
    nb = ctypes.c_size_t(0)
    assert lib.kvsel_score(None, None, 1, 8, 4, 128, 4096, 32, 0, 0, 0.088, 7, None, None, None,
                           None, None) == ARG
    # non-null workspace but null inputs -> ARG; too small -> WORKSPACE (pointers unused)
    fake = ctypes.c_void_p(1 << 20)
    nb.value = 1 << 30
    assert lib.kvsel_score(None, None, 1, 8, 4, 128, 4096, 32, 0, 0, 0.088, 7, None, None, fake,
                           ctypes.byref(nb), None) == ARG
    nb.value = 16
    assert lib.kvsel_score(fake, fake, 1, 8, 4, 128, 4096, 32, 0, 0, 0.088, 7, fake, None, fake,
                           ctypes.byref(nb), None) == WS
    nb.value = 1 << 30
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert lib.kvsel_score(odd, fake, 1, 8, 4, 128, 4096, 32, 0, 0, 0.088, 7, fake, None, fake,
                           ctypes.byref(nb), None) == ARG


def _select(lib, weight=False, **kw):
    a = dict(L=1, H=8, n=4096, W=32, budget=819, adaptive=0, norm=1.0, eps=1e-4, alpha=0.5)
    a.update(kw)
    nb = ctypes.c_size_t(0)
    w = ctypes.c_void_p(1 << 20) if weight else None
    return lib.kvsel_select(None, w, a["L"], a["H"], a["n"], a["W"], a["budget"], a["adaptive"],
                            a["norm"], a["eps"], a["alpha"], None, None, None, None,
                            ctypes.byref(nb), None)


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(budget=32), OK), (dict(budget=4096), OK), (dict(W=0, budget=0), OK),
    (dict(budget=31), ARG), (dict(budget=4097), ARG), (dict(W=4096), ARG), (dict(W=-1), ARG),
    (dict(adaptive=2), ARG), (dict(adaptive=1, budget=255), ARG), (dict(adaptive=1, budget=256), OK),
    (dict(adaptive=1, budget=8 * 4096), OK), (dict(adaptive=1, budget=8 * 4096 + 1), ARG),
    (dict(L=0), ARG), (dict(H=0), ARG), (dict(n=0), ARG),
])
def test_select_ranges(lib, kw, code):
    assert _select(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(alpha=-0.1), ARG), (dict(alpha=1.5), ARG), (dict(alpha=float("nan")), ARG),
    (dict(norm=0.0), ARG), (dict(eps=-1.0), ARG), (dict(eps=float("inf")), ARG), (dict(), OK),
])
@no_gpu_only
def test_select_two_stage_ranges(lib, kw, code):
    assert _select(lib, weight=True, **kw) == code


@no_gpu_only
def test_value_weight_and_compact_reject(lib):
    p = ctypes.c_void_p(1 << 20)
    f = lib.kvsel_value_weight
    nb = ctypes.c_size_t(1 << 30)
    ws = ctypes.byref(nb)
    assert f(None, p, 1, 8, 4, 128, 100, 4096, 68, 0, p, p, ws, None) == ARG
    assert f(p, p, 1, 8, 4, 128, 100, 4096, 101, 0, p, p, ws, None) == ARG    # n_cand > n
    assert f(p, p, 1, 8, 4, 128, 100, 4096, 0, 0, p, p, ws, None) == ARG
    assert f(p, p, 1, 8, 4, 128, 100, 4096, 68, 2, p, p, ws, None) == ARG     # group mode
    assert f(p, p, 1, 8, 4, 128, 100, 4096, 68, -1, p, p, ws, None) == ARG
    assert f(p, p, 1, 8, 4, 128, 100, 4096, 68, 0, p, p, None, None) == ARG   # no ws_bytes
    assert f(p, p, 1, 8, 4, 64, 100, 4096, 68, 0, p, p, ws, None) == UNSUP
    assert f(p, p, 1, 8, 4, 128, 100, 4010, 68, 0, p, p, ws, None) == UNSUP   # D % 32
    assert f(p, p, 1, 8, 4, 128, 100, 1 << 18, 68, 0, p, p, ws, None) == UNSUP  # w_o of 2^31 bytes
    small = ctypes.c_size_t(1000)
    assert f(p, p, 2, 8, 4, 128, 100, 4096, 68, 1, p, p, ctypes.byref(small), None) == WS
    assert f(p, p, 1, 8, 4, 128, 100, 4096, 68, 1, p, ctypes.c_void_p((1 << 20) + 8), ws, None) == ARG
    c = lib.kvsel_compact
    assert c(None, p, 1, 8, 128, 100, p, None, 16, p, p, None) == ARG
    assert c(p, p, 1, 8, 128, 100, p, None, 12, p, p, None) == ARG  # not divisible by H
    assert c(p, p, 1, 8, 128, 100, p, None, 808, p, p, None) == ARG  # more rows than the cache
    assert c(p, p, 1, 8, 12, 100, p, None, 16, p, p, None) == UNSUP


def test_value_weight_workspace_query(lib):
    nb = ctypes.c_size_t(123)
    f = lib.kvsel_value_weight
    # group mode 0 needs none; mode 1 holds the group-summed slices of every layer
    assert f(None, None, 2, 8, 4, 128, 100, 4096, 68, 0, None, None, ctypes.byref(nb), None) == OK
    assert nb.value == 0
    assert f(None, None, 2, 8, 4, 128, 100, 4096, 68, 1, None, None, ctypes.byref(nb), None) == OK
    assert nb.value == 2 * 4096 * 8 * 128 * 2


def _decode(lib, **kw):
    a = dict(L=2, H=8, G=4, d=128, kept=800, offs=None, scale=0.088)
    a.update(kw)
    nb = ctypes.c_size_t(0)
    return lib.kvsel_decode_attention(None, None, None, a["L"], a["H"], a["G"], a["d"], a["kept"],
                                      a["offs"], a["scale"], None, None, ctypes.byref(nb), None), nb.value


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(G=8), OK), (dict(G=1), OK), (dict(L=0), ARG), (dict(H=0), ARG),
    (dict(G=0), ARG), (dict(kept=0), ARG), (dict(kept=801), ARG), (dict(scale=0.0), ARG),
    (dict(scale=float("nan")), ARG), (dict(G=9), UNSUP), (dict(d=64), UNSUP),
    (dict(H=1025, kept=1025 * 4), UNSUP),
])
def test_decode_ranges(lib, kw, code):
    assert _decode(lib, **kw)[0] == code


def test_decode_workspace_query(lib):
    rc, nb = _decode(lib)
    assert rc == OK and nb > 0
    # ragged heads (offsets given) size for the worst split of the rows
    rc2, nb2 = _decode(lib, kept=801, offs=ctypes.c_void_p(1 << 20))
    assert rc2 == OK and nb2 >= nb


def _l2_args(**kw):
    a = dict(L=2, H=8, G=4, d=128, n=100, D=4096, n_cand=68)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), ARG), (dict(G=0), ARG), (dict(D=0), ARG), (dict(d=64), UNSUP),
    (dict(H=1 << 20, G=16), UNSUP),
])
@no_gpu_only
def test_value_l2_factor_reject(lib, kw, code):
    p = ctypes.c_void_p(1 << 20)
    a = _l2_args(**kw)
    assert lib.kvsel_value_l2_factor(p, a["L"], a["H"], a["G"], a["d"], a["D"], p, None) == code


@no_gpu_only
def test_value_l2_factor_pointers(lib):
    p = ctypes.c_void_p(1 << 20)
    f = lib.kvsel_value_l2_factor
    assert f(None, 2, 8, 4, 128, 4096, p, None) == ARG
    assert f(p, 2, 8, 4, 128, 4096, None, None) == ARG
    assert f(p, 2, 8, 4, 128, 4096, ctypes.c_void_p((1 << 20) + 8), None) == ARG   # misaligned


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), ARG), (dict(G=0), ARG), (dict(n_cand=0), ARG), (dict(n_cand=101), ARG),
    (dict(n=0), ARG), (dict(d=64), UNSUP),
])
@no_gpu_only
def test_value_weight_l2_reject(lib, kw, code):
    p = ctypes.c_void_p(1 << 20)
    a = _l2_args(**kw)
    assert lib.kvsel_value_weight_l2(p, p, a["L"], a["H"], a["G"], a["d"], a["n"], a["n_cand"],
                                     p, None) == code


@no_gpu_only
def test_value_weight_l2_pointers(lib):
    p = ctypes.c_void_p(1 << 20)
    f = lib.kvsel_value_weight_l2
    assert f(None, p, 2, 8, 4, 128, 100, 68, p, None) == ARG
    assert f(p, None, 2, 8, 4, 128, 100, 68, p, None) == ARG
    assert f(p, p, 2, 8, 4, 128, 100, 68, None, None) == ARG
    assert f(p, ctypes.c_void_p((1 << 20) + 8), 2, 8, 4, 128, 100, 68, p, None) == ARG


def _sel_budgets(lib, weight=False, **kw):
    a = dict(L=2, H=8, n=1000, W=32, stride=4000, alpha=0.5, norm=0.01, eps=1e-4)
    a.update(kw)
    nb = ctypes.c_size_t(0)
    w = ctypes.c_void_p(1 << 20) if weight else None
    return lib.kvsel_select_budgets(None, w, a["L"], a["H"], a["n"], a["W"], None, a["stride"],
                                    a["norm"], a["eps"], a["alpha"], None, None, None, None,
                                    ctypes.byref(nb), None), nb.value


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(W=0), OK), (dict(stride=1), OK), (dict(stride=8000), OK),
    (dict(n=50000), OK), (dict(L=0), ARG), (dict(H=0), ARG), (dict(W=1000), ARG),
    (dict(W=-1), ARG), (dict(stride=0), ARG), (dict(stride=8001), ARG),
    (dict(H=1 << 16, n=1 << 16, stride=5), UNSUP),
])
def test_select_budgets_ranges(lib, kw, code):
    assert _sel_budgets(lib, **kw)[0] == code


@pytest.mark.parametrize("kw,code", [
    (dict(alpha=-0.1), ARG), (dict(alpha=1.5), ARG), (dict(norm=0.0), ARG),
    (dict(eps=-1.0), ARG), (dict(alpha=1.0), OK),
])
def test_select_budgets_two_stage_ranges(lib, kw, code):
    assert _sel_budgets(lib, weight=True, **kw)[0] == code


def test_select_budgets_workspace_like_select(lib):
    # the same segments as the per-head select: the same workspace
    rc, nb = _sel_budgets(lib, n=50000, W=32)
    nb2 = ctypes.c_size_t(0)
    rc2 = lib.kvsel_select(None, None, 2, 8, 50000, 32, 5000, 0, 1.0, 1e-4, 0.5, None, None, None,
                           None, ctypes.byref(nb2), None)
    assert rc == OK and rc2 == OK and nb == nb2.value > 0


@no_gpu_only
def test_select_budgets_pointers(lib):
    p = ctypes.c_void_p(1 << 20)
    f = lib.kvsel_select_budgets
    nb = ctypes.c_size_t(1 << 20)
    args = lambda sc, bud, idx, offs: (sc, None, 2, 8, 1000, 32, bud, 4000, 0.01, 1e-4, 0.5, idx,
                                       offs, None, p, ctypes.byref(nb), None)
    assert f(*args(None, p, p, p)) == ARG
    assert f(*args(p, None, p, p)) == ARG
    assert f(*args(p, p, None, p)) == ARG
    assert f(*args(p, p, p, None)) == ARG


def test_score_logit_mode(lib):
    assert _score(lib, mode=1, agg=2)[0] == OK
    assert _score(lib, mode=0, agg=2)[0] == ARG      # external queries only
    assert _score(lib, mode=1, agg=3)[0] == ARG
    # no pass 1: a smaller workspace than the softmax max of the same shape
    assert _score(lib, mode=1, agg=2, W=4096)[1] < _score(lib, mode=1, agg=1, W=4096)[1]


def _head_budgets(lib, **kw):
    a = dict(L=4, H=8, keep=10, n=1000, W=32)
    a.update(kw)
    nb = ctypes.c_size_t(0)
    rc = lib.kvsel_head_budgets(None, a["L"], a["H"], a["keep"], a["n"], a["W"], None, None,
                                ctypes.byref(nb), None)
    return rc, nb.value


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(keep=0), OK), (dict(keep=32), OK), (dict(W=0), OK), (dict(W=1000), OK),
    (dict(L=100, H=400, keep=20000), OK),   # more heads than one workgroup holds
    (dict(keep=33), ARG), (dict(keep=-1), ARG), (dict(W=1001), ARG), (dict(W=-1), ARG),
    (dict(L=0), ARG), (dict(n=0), ARG),
])
def test_head_budgets_ranges(lib, kw, code):
    assert _head_budgets(lib, **kw)[0] == code


@no_gpu_only
def test_head_score_and_budgets_pointers(lib):
    p = ctypes.c_void_p(1 << 20)
    assert lib.kvsel_head_score(None, 2, 8, 100, p, None) == ARG
    assert lib.kvsel_head_score(p, 2, 8, 100, None, None) == ARG
    assert lib.kvsel_head_score(p, 0, 8, 100, p, None) == ARG
    assert lib.kvsel_head_score(p, 2, 8, 0, p, None) == ARG
    nb = ctypes.c_size_t(1 << 20)
    f = lib.kvsel_head_budgets
    assert f(None, 2, 8, 3, 100, 8, p, p, ctypes.byref(nb), None) == ARG
    assert f(p, 2, 8, 3, 100, 8, None, p, ctypes.byref(nb), None) == ARG
    small = ctypes.c_size_t(1)
    assert f(p, 2, 8, 3, 100, 8, p, p, ctypes.byref(small), None) == WS


def _chunked(lib, **kw):
    a = dict(L=2, H=4, G=7, d=128, n=32768, m=2048, npr=32, scale=0.088, pool=1)
    a.update(kw)
    nb = ctypes.c_size_t(0)
    rc = lib.kvsel_score_chunked(None, None, None, a["L"], a["H"], a["G"], a["d"], a["n"], a["m"],
                                 a["npr"], a["scale"], a["pool"], None, None, None,
                                 ctypes.byref(nb), None)
    return rc, nb.value


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(npr=0), OK), (dict(m=1), OK), (dict(m=100000), OK), (dict(pool=5), OK),
    (dict(m=0), ARG), (dict(npr=-1), ARG), (dict(pool=2), ARG), (dict(scale=0.0), ARG),
    (dict(L=0), ARG), (dict(d=64), UNSUP), (dict(pool=67), UNSUP),
    (dict(G=64, m=32768, npr=100000), UNSUP),   # a head's query rows past 2^31 bytes
])
def test_score_chunked_ranges(lib, kw, code):
    assert _chunked(lib, **kw)[0] == code


def test_score_chunked_workspace(lib):
    # m past n is one chunk: the same plan as m == n
    assert _chunked(lib, n=5000, m=100000)[1] == _chunked(lib, n=5000, m=5000)[1]


@no_gpu_only
def test_score_chunked_pointers(lib):
    p = ctypes.c_void_p(1 << 20)
    nb = ctypes.c_size_t(1 << 30)
    f = lib.kvsel_score_chunked
    base = (2, 4, 7, 128, 32768, 2048, 32, 0.088, 1)
    assert f(p, p, None, *base, p, None, p, ctypes.byref(nb), None) == ARG
    assert f(None, p, p, *base, p, None, p, ctypes.byref(nb), None) == ARG
    assert f(p, p, p, *base, None, None, p, ctypes.byref(nb), None) == ARG


def _anchor_sel(lib, **kw):
    a = dict(L=2, H=8, n=4096, W=32, k=64, rho=0.7)
    a.update(kw)
    nb = ctypes.c_size_t(0)
    return lib.kvsel_anchor_select(None, None, a["L"], a["H"], a["n"], a["W"], a["k"], a["rho"],
                                   None, None, ctypes.byref(nb), None), nb.value


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(k=32), OK), (dict(k=4096), OK), (dict(rho=0.0), OK), (dict(rho=1.0), OK),
    (dict(W=0, k=0), OK), (dict(n=50000, k=390), OK),
    (dict(k=31), ARG), (dict(k=4097), ARG), (dict(rho=1.5), ARG), (dict(rho=-0.1), ARG),
    (dict(W=4096), ARG), (dict(L=0), ARG),
])
def test_anchor_select_ranges(lib, kw, code):
    assert _anchor_sel(lib, **kw)[0] == code


def _anchor_asg(lib, **kw):
    a = dict(L=2, H=8, d=128, n=4096, k=32)
    a.update(kw)
    nb = ctypes.c_size_t(0)
    return lib.kvsel_anchor_assign(None, None, a["L"], a["H"], a["d"], a["n"], a["k"], None, None,
                                   None, ctypes.byref(nb), None), nb.value


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(k=1), OK), (dict(k=2048, n=300000), OK), (dict(k=4096), UNSUP),
    (dict(k=0), ARG), (dict(k=5000), ARG), (dict(n=0), ARG), (dict(d=64), UNSUP),
    (dict(k=2049, n=300000), UNSUP), (dict(L=300, H=300), UNSUP),
])
def test_anchor_assign_ranges(lib, kw, code):
    rc, nb = _anchor_asg(lib, **kw)
    assert rc == code


def test_anchor_assign_workspace(lib):
    # the gathered anchor rows (k rounded up to 64) and one float per anchor
    rc, nb = _anchor_asg(lib, L=2, H=8, k=100)
    assert rc == OK and nb >= 2 * 8 * 128 * (256 + 4)


@no_gpu_only
def test_anchor_pointers(lib):
    p = ctypes.c_void_p(1 << 20)
    nb = ctypes.c_size_t(1 << 30)
    f = lib.kvsel_anchor_select
    assert f(None, p, 2, 8, 4096, 32, 64, 0.7, p, p, ctypes.byref(nb), None) == ARG
    assert f(p, None, 2, 8, 4096, 32, 64, 0.7, p, p, ctypes.byref(nb), None) == ARG
    assert f(p, p, 2, 8, 4096, 32, 64, 0.7, None, p, ctypes.byref(nb), None) == ARG
    g = lib.kvsel_anchor_assign
    assert g(None, p, 2, 8, 128, 4096, 32, p, p, p, ctypes.byref(nb), None) == ARG
    assert g(p, None, 2, 8, 128, 4096, 32, p, p, p, ctypes.byref(nb), None) == ARG
    assert g(p, p, 2, 8, 128, 4096, 32, None, p, p, ctypes.byref(nb), None) == ARG
    small = ctypes.c_size_t(16)
    assert g(p, p, 2, 8, 128, 4096, 32, p, p, p, ctypes.byref(small), None) == WS
