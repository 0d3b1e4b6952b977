"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import math
import os
import re

import pytest

from attention_space_retrieval_amd import kvs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvs.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kvs.load()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) == 22
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(kvs.ENTRY_POINTS) == names


def test_status_strings(lib):
    assert lib.kvs_status_string(0) == b"ok"
    assert lib.kvs_status_string(5) == b"workspace missing or too small"
    assert lib.kvs_version() >= 100


FAKE = 0x1000   # never dereferenced: every call below must be rejected on the host


def test_qmem_rejections(lib):
    f = lib.kvs_qmem_update
    assert f(None, 1, 2, 4, 8, 128, 0.5, 1, FAKE, None) == 1
    assert f(FAKE, 7, 2, 4, 8, 128, 0.5, 1, FAKE, None) == 3
    assert f(FAKE, 1, 2, 4, 0, 128, 0.5, 1, FAKE, None) == 1
    assert f(FAKE, 1, 2, 4, 8, 128, -1.0, 1, FAKE, None) == 1
    assert f(FAKE, 1, 2, 4, 8, 128, math.nan, 1, FAKE, None) == 1
    assert f(FAKE, 1, 2, 4, 8, 96, 0.5, 1, FAKE, None) == 4


def test_rule_rejections(lib):
    f = lib.kvs_rule_score
    ws = lib.kvs_rule_score_workspace(2, 4, 2, 1024)
    assert ws >= 2 * 4 * 1024 * 4
    args = dict(K=FAKE, dt=1, M=FAKE, L=2, Hq=4, Hkv=2, D=128, N=1024, pi=16, qs=992, qe=1024,
                rule=FAKE, ws=FAKE, wsb=ws)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["K"], a["dt"], a["M"], a["L"], a["Hq"], a["Hkv"], a["D"], a["N"], a["pi"],
                 a["qs"], a["qe"], a["rule"], a["ws"], a["wsb"], None)

    assert call(K=None) == 1
    assert call(dt=5) == 3
    assert call(Hq=5) == 2
    assert call(qs=10, qe=5) == 1
    assert call(pi=-1) == 1
    assert call(D=80) == 4
    assert call(Hq=34, Hkv=2) == 4          # G = 17 > 16 is not built
    assert call(ws=None) == 5
    assert call(wsb=ws - 1) == 5
    assert call(N=1 << 31) == 2
    assert call(N=0) == 0                   # empty input: nothing to do, nothing launched
    assert call(N=0, K=None, rule=None) == 0   # an empty tensor may come as NULL
    assert call(K=None) == 1 and call(rule=None) == 1


def test_topk_slot_meank_rerope_rejections(lib):
    assert lib.kvs_topk_select(None, 10, 0, 1, 5, 6, 3, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert lib.kvs_topk_select(FAKE, 10, 3, 1, 5, 6, 3, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert lib.kvs_topk_select(FAKE, 10, 0, 1, 5, 6, -1, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert lib.kvs_topk_select(FAKE, 1 << 31, 0, 1, 5, 6, 3, FAKE, FAKE, FAKE, None, 0, None) == 2
    # up to 32768 scores no workspace; beyond, an optional one (too small is an error)
    assert lib.kvs_topk_workspace(32768) == 0
    need = lib.kvs_topk_workspace(92160)
    assert need >= 4 * (256 + 2 * 45)
    assert lib.kvs_topk_select(FAKE, 92160, 0, 64, 92096, 92160, 8192, FAKE, FAKE, FAKE, FAKE, need - 1,
                               None) == 5
    # the fused redirect: the same checks, and both slot arrays when n > 0
    R = lib.kvs_topk_select_redirect
    assert R(None, 10, 0, 1, 5, 6, 3, FAKE, FAKE, FAKE, FAKE, -1, FAKE, None, 0, None) == 1
    assert R(FAKE, 10, 0, 1, 5, 6, 3, FAKE, FAKE, FAKE, None, -1, FAKE, None, 0, None) == 1
    assert R(FAKE, 10, 0, 1, 5, 6, 3, FAKE, FAKE, FAKE, FAKE, -1, None, None, 0, None) == 1
    assert R(FAKE, 1 << 31, 0, 1, 5, 6, 3, FAKE, FAKE, FAKE, FAKE, -1, FAKE, None, 0, None) == 2
    assert R(FAKE, 92160, 0, 64, 92096, 92160, 8192, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, need - 1, None) == 5
    # the no-allocation variant: same checks, and a fixed size limit instead of a workspace
    nmax = lib.kvs_topk_noalloc_max()
    assert nmax == 1 << 24
    assert lib.kvs_topk_select_noalloc(FAKE, nmax + 1, 0, 64, nmax - 64, nmax, 8192, FAKE, FAKE, FAKE,
                                       None) == 7
    assert lib.kvs_topk_select_noalloc(None, 10, 0, 1, 5, 6, 3, FAKE, FAKE, FAKE, None) == 1
    assert lib.kvs_topk_select_noalloc(FAKE, 10, 0, 1, 5, 6, -1, FAKE, FAKE, FAKE, None) == 1
    assert lib.kvs_topk_select_noalloc(FAKE, 1 << 31, 0, 1, 5, 6, 3, FAKE, FAKE, FAKE, None) == 2
    assert lib.kvs_status_string(7) == b"size above the fixed limit of a no-allocation entry point"
    assert lib.kvs_slotmap_redirect(None, FAKE, 10, -1, FAKE, None) == 1
    assert lib.kvs_slotmap_redirect(FAKE, FAKE, -1, -1, FAKE, None) == 1
    assert lib.kvs_meank_build(FAKE, 2, 2, 128, 64, 16, 0, 0, 1e6, None, FAKE, None) == 4
    assert lib.kvs_meank_build(FAKE, 2, 2, 128, 64, 32, 1, 0, math.inf, None, FAKE, None) == 1
    assert lib.kvs_meank_build(FAKE, 2, 2, 128, 64, 32, 1, -5, 1e6, None, FAKE, None) == 1
    assert lib.kvs_meank_build(None, 2, 2, 128, 64, 32, 0, 0, 1e6, None, FAKE, None) == 1
    a = lib.kvs_meank_append
    assert a(FAKE, 2, 2, 128, 40, 30, 0, 1e6, FAKE, 64, FAKE, None) == 2      # t0 + n_new > cap
    assert a(FAKE, 2, 2, 128, -1, 30, 0, 1e6, FAKE, 64, FAKE, None) == 1
    assert a(FAKE, 2, 2, 128, 0, 30, 0, 0.0, FAKE, 64, FAKE, None) == 1       # theta
    assert a(FAKE, 2, 2, 96, 0, 30, 0, 1e6, FAKE, 64, FAKE, None) == 4
    assert a(None, 2, 2, 128, 0, 30, 0, 1e6, FAKE, 64, FAKE, None) == 1
    assert a(None, 2, 2, 128, 10, 0, 0, 1e6, None, 64, None, None) == 0       # empty chunk: no-op
    ws = lib.kvs_meank_score_workspace(2, 8, 2, 50, 300)
    assert ws > 0
    assert lib.kvs_meank_score(FAKE, FAKE, 2, 8, 2, 96, 50, 300, 4, 7, FAKE, FAKE, ws, None) == 4
    assert lib.kvs_meank_score(FAKE, FAKE, 2, 8, 3, 128, 50, 300, 4, 7, FAKE, FAKE, ws, None) == 2
    assert lib.kvs_meank_score(FAKE, FAKE, 2, 8, 2, 128, 50, 300, 4, 7, FAKE, FAKE, ws - 1, None) == 5
    assert lib.kvs_meank_score(FAKE, FAKE, 2, 8, 2, 128, 50, 300, -1, 7, FAKE, FAKE, ws, None) == 1
    r = lib.kvs_rerope_scatter
    assert r(FAKE, FAKE, 640, FAKE, None, 3, 2, 2, 128, 32, 0, 1e6, FAKE, None, 8, None, None) == 1
    assert r(FAKE, FAKE, 650, FAKE, None, 3, 2, 2, 128, 32, 0, 1e6, FAKE, FAKE, 8, None, None) == 2
    assert r(FAKE, FAKE, 640, FAKE, None, 3, 2, 2, 128, 64, 0, 1e6, FAKE, FAKE, 8, None, None) == 4
    assert r(FAKE, FAKE, 640, FAKE, None, 3, 2, 2, 128, 32, 0, -1.0, FAKE, FAKE, 8, None, None) == 1
    assert r(FAKE, FAKE, 640, None, None, 3, 2, 2, 128, 32, 0, 1e6, FAKE, FAKE, 8, None, None) == 1


def test_rule_paged_rejections(lib):
    f = lib.kvs_rule_score_paged
    ws = lib.kvs_rule_score_workspace(2, 4, 2, 1024)
    ok = [FAKE, 1, FAKE, 2048, FAKE, 2, 4, 2, 128, 1024, 16, 992, 1024, FAKE, FAKE, ws, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a2=None) == 1            # no slot map
    assert call(a3=0) == 1               # empty pool
    assert call(a1=5) == 3               # dtype
    assert call(a7=3) == 2               # H_q % H_kv
    assert call(a8=96) == 4
    assert call(a15=ws - 1) == 5


def test_window_rejections(lib):
    f = lib.kvs_window_score
    ws = lib.kvs_window_score_workspace(2, 8, 2, 16, 1000)
    assert ws > 0
    assert f(FAKE, FAKE, 2, 8, 2, 128, 1000, 0, 4, 990, 1000, FAKE, FAKE, ws, None) == 1      # W = 0
    assert f(FAKE, FAKE, 2, 8, 3, 128, 1000, 16, 4, 990, 1000, FAKE, FAKE, ws, None) == 2
    assert f(FAKE, FAKE, 2, 8, 2, 96, 1000, 16, 4, 990, 1000, FAKE, FAKE, ws, None) == 4
    assert f(FAKE, FAKE, 2, 8, 2, 128, 1000, 16, 4, 990, 1000, FAKE, FAKE, ws - 1, None) == 5
    assert f(None, FAKE, 2, 8, 2, 128, 1000, 16, 4, 990, 1000, FAKE, FAKE, ws, None) == 1


def test_working_set_rejections(lib):
    f = lib.kvs_working_set_update
    ws = lib.kvs_working_set_workspace(8)
    assert ws >= 8 * 4
    base = [FAKE, FAKE, 640, FAKE, FAKE, 3, FAKE, 4, 2, 2, 128, 32, 0, 1e6, FAKE, FAKE, 8,
            FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a7=9) == 2                 # more selected blocks than pool pages
    assert call(a2=650) == 2               # src_tokens not a multiple of 32
    assert call(a11=16) == 4               # block size
    assert call(a10=96) == 4               # head dim
    assert call(a13=-1.0) == 1             # theta
    assert call(a0=None) == 1
    assert call(a1=None) == 1              # V source without V pool
    assert call(a20=None) == 1             # counts
    assert call(a23=ws - 1) == 5
    assert call(a6=None) == 1              # new blocks missing while n_new > 0


def test_oversized_launches_are_rejected(lib):
    r = lib.kvs_rerope_scatter
    assert r(FAKE, None, 640, FAKE, None, 1 << 24, 2, 2, 128, 32, 0, 1e6, FAKE, None, 8, None, None) == 2
    # one workgroup per (block, 16 slices): 2^22 blocks over 64 slices is 2^24 workgroups
    assert r(FAKE, None, 640, FAKE, None, 1 << 22, 8, 8, 128, 32, 0, 1e6, FAKE, None, 8, None, None) == 2
    ws = 1 << 30
    assert lib.kvs_meank_score(FAKE, FAKE, 4, 8, 2, 128, 50, (1 << 31) - 1, 4, 7, FAKE, FAKE, ws, None) == 2
    # streamed operands past 2^23 - 128 rows (32-bit buffer offsets): index blocks, query rows, keys, window rows
    big = (1 << 23) - 127
    assert lib.kvs_meank_score(FAKE, FAKE, 1, 2, 2, 128, 4, big, 4, 7, FAKE, FAKE, ws, None) == 2
    assert lib.kvs_meank_score(FAKE, FAKE, 1, 2, 1, 128, big // 2 + 1, 1000, 4, 7, FAKE, FAKE, ws, None) == 2
    assert lib.kvs_window_score(FAKE, FAKE, 1, 2, 2, 128, big, 4, 4, 0, 0, FAKE, FAKE, ws, None) == 2
    assert lib.kvs_window_score(FAKE, FAKE, 1, 2, 1, 128, 1000, big // 2 + 1, 4, 0, 0, FAKE, FAKE, ws, None) == 2


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU"):
        kvs.kvs_rule_score(torch.zeros(1, 1, 8, 64), torch.zeros(1, 1, 64), 0, 0, 0)
    with pytest.raises(ValueError, match="GPU"):
        kvs.kvs_topk_select(torch.zeros(8), (0, 0), (0, 0), 3)
