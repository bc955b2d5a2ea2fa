"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, and rejects bad arguments before launching anything
(every call below fails validation, so no kernel is ever enqueued)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsa.h")
LIB = os.path.join(ROOT, "block_sparse_attention_hilbert3d_amd", "libhsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libhsa.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_five_steps():
    names = _declared()
    for n in ["hsa_plan", "hsa_perm", "hsa_score", "hsa_select", "hsa_attn", "hsa_unperm"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (hsa_[a-z_0-9]+)$", out, flags=re.M))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    L = ctypes.CDLL(LIB)
    for n in _declared():
        assert getattr(L, n) is not None


@pytest.fixture(scope="module")
def B():
    from block_sparse_attention_hilbert3d_amd import binding
    return binding


def _err(B, status):
    return status, B.lib().hsa_last_error().decode()


def test_version_and_strings(B):
    L = B.lib()
    assert L.hsa_abi_version() == 4
    assert L.hsa_status_str(0) == b"ok"
    assert L.hsa_status_str(5) == b"workspace too small"


def test_plan_size_closed_forms(B):
    assert B.hsa_plan_size(21, 30, 52, "hilbert", 128) == (32768, 256)
    assert B.hsa_plan_size(61, 30, 52, "frame", 128) == (101504, 793)
    assert B.hsa_plan_size(33, 45, 80, "hilbert", 128) == (118912, 929)
    assert B.hsa_plan_size(4, 8, 8, "row", 64) == (256, 4)
    with pytest.raises(B.HsaError):
        B.hsa_plan_size(0, 8, 8, "row", 64)
    with pytest.raises(B.HsaError):
        B.hsa_plan_size(2000, 8, 8, "row", 64)


def test_plan_workspace_sizes(B):
    L = B.lib()
    assert L.hsa_plan_ws_size(21, 30, 52, 0) == 0
    assert L.hsa_plan_ws_size(21, 30, 52, 1) == (64 ** 3 // 2048) * 4
    assert L.hsa_plan_ws_size(33, 45, 80, 1) == (128 ** 3 // 2048) * 4


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
NULL = ctypes.c_void_p(0)


def test_perm_validation(B):
    L = B.lib()
    arr = (ctypes.c_void_p * 3)(FAKE.value, FAKE.value, FAKE.value)
    P = (0, NULL)                                                                  # no pooling
    assert L.hsa_perm(4, arr, arr, FAKE, 10, 16, 2, 64, 128, 1, *P, NULL) == 6          # n_tensors
    assert L.hsa_perm(1, arr, arr, NULL, 10, 16, 2, 64, 128, 1, *P, NULL) == 1          # perm
    assert L.hsa_perm(1, arr, arr, FAKE, 10, 16, 2, 96, 192, 1, *P, NULL) == 4          # D
    assert L.hsa_perm(1, arr, arr, FAKE, 10, 16, 2, 64, 128, 7, *P, NULL) == 3          # dtype
    assert L.hsa_perm(1, arr, arr, FAKE, 20, 16, 2, 64, 128, 1, *P, NULL) == 2          # n_pad < N
    assert L.hsa_perm(1, arr, arr, FAKE, 10, 16, 2, 64, 100, 1, *P, NULL) == 2          # stride < nh*D
    assert L.hsa_perm(1, arr, arr, FAKE, 10, 16, 2, 64, 132, 1, *P, NULL) == 6          # stride alignment
    assert L.hsa_perm(1, arr, arr, FAKE, 10, 16, 200, 64, 12800, 1, *P, NULL) == 4      # row > 16 KB
    bad = (ctypes.c_void_p * 1)(0x10004)
    assert L.hsa_perm(1, bad, arr, FAKE, 10, 16, 2, 64, 128, 1, *P, NULL) == 6          # pointer alignment
    assert b"aligned" in L.hsa_last_error()
    assert L.hsa_perm(2, arr, arr, FAKE, 10, 16, 2, 64, 128, 1, 24, FAKE, NULL) == 4    # pool_s
    assert L.hsa_perm(2, arr, arr, FAKE, 10, 24, 2, 64, 128, 1, 16, FAKE, NULL) == 2    # pool_s | n_pad
    assert L.hsa_perm(1, arr, arr, FAKE, 10, 16, 2, 64, 128, 1, 16, FAKE, NULL) == 6    # needs Q and K
    # a null output is a pooled-only tensor: allowed for tensors 0 and 1 when pooling, never else
    some_null = (ctypes.c_void_p * 3)(None, FAKE.value, FAKE.value)
    assert L.hsa_perm(3, arr, some_null, FAKE, 10, 16, 2, 64, 128, 1, *P, NULL) == 1
    last_null = (ctypes.c_void_p * 3)(FAKE.value, FAKE.value, None)
    assert L.hsa_perm(3, arr, last_null, FAKE, 10, 16, 2, 64, 128, 1, 16, FAKE, NULL) == 1


def test_score_validation(B):
    L = B.lib()
    ws_n = L.hsa_score_ws_size(2, 256, 16, 64)
    assert ws_n > 0
    args = lambda **kw: dict(dict(nh=2, nb=4, Bs=64, s=16, D=64, dt=1, agg=0, scale=0.125,
                                  ws=FAKE, wsn=ws_n), **kw)

    def call(a):
        return L.hsa_score(FAKE, FAKE, NULL, FAKE, a["nh"], a["nb"], a["Bs"], a["s"], a["D"],
                           a["dt"], a["agg"], a["scale"], FAKE, a["ws"], a["wsn"], NULL)
    assert call(args(s=24)) == 4
    assert call(args(Bs=64, s=128)) == 2
    assert call(args(agg=5)) == 6
    assert call(args(scale=-1.0)) == 6
    assert call(args(wsn=ws_n - 1)) == 5
    assert call(args(ws=NULL)) == 5
    assert call(args(nb=140000, Bs=128, s=16)) == 4     # more than 2^20 sub-blocks per head
    assert L.hsa_score(NULL, FAKE, NULL, FAKE, 2, 4, 64, 16, 64, 1, 0, 0.125, FAKE, FAKE, ws_n, NULL) == 1
    # with pooled means the workspace is not needed, but S must still be valid
    assert L.hsa_score(NULL, NULL, FAKE, FAKE, 2, 4, 64, 16, 64, 1, 0, 0.125, NULL, NULL, 0, NULL) == 1
    assert L.hsa_score(NULL, NULL, ctypes.c_void_p(0x10008), FAKE, 2, 4, 64, 16, 64, 1, 0, 0.125, FAKE, NULL, 0, NULL) == 6


def test_select_validation(B):
    L = B.lib()
    p = B.make_params("topk", k=5)
    assert L.hsa_select(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 8, NULL, 0, NULL) == 6     # k > nb
    p = B.make_params("topk", k=3)
    assert L.hsa_select(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 2, NULL, 0, NULL) == 2     # max_kv < k
    assert L.hsa_select(NULL, 2, 4, ctypes.byref(p), FAKE, FAKE, 4, NULL, 0, NULL) == 1
    p = B.make_params("thresh_global", tau=0.25, budget_ratio=0.3)
    n = L.hsa_select_ws_size(2, 4, ctypes.byref(p))
    assert n > 0
    assert L.hsa_select(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 3, FAKE, n, NULL) == 2     # max_kv != nb
    assert L.hsa_select(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 4, FAKE, n - 1, NULL) == 5
    p = B.make_params("thresh_global", tau=0.25, budget_ratio=1.5)
    assert L.hsa_select(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 4, FAKE, n, NULL) == 6
    # tau * 2^62 must fit 64 bits: 4 is refused, the largest double below it is not
    p = B.make_params("thresh_global", tau=4.0, budget_ratio=0.3)
    assert L.hsa_select(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 4, FAKE, n, NULL) == 6
    p = B.make_params("thresh_global", tau=float.fromhex("0x1.fffffffffffffp+1"), budget_ratio=0.3)
    assert L.hsa_select(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 3, FAKE, n, NULL) == 2     # passes tau
    p = B.make_params("lvsa", frames=61, tiles_per_frame=13, C=21, T_per=8, step=0)
    assert L.hsa_select(NULL, 12, 793, ctypes.byref(p), FAKE, FAKE, 21 * 13 - 1, NULL, 0, NULL) == 2
    p = B.make_params("lvsa", frames=61, tiles_per_frame=13, C=21, T_per=8, step=0)
    assert L.hsa_select(NULL, 12, 792, ctypes.byref(p), FAKE, FAKE, 21 * 13, NULL, 0, NULL) == 2
    p = B.make_params("lvsa", frames=61, tiles_per_frame=13, C=0, T_per=8, step=0)
    assert L.hsa_select(NULL, 12, 793, ctypes.byref(p), FAKE, FAKE, 21 * 13, NULL, 0, NULL) == 6
    p = B.SelectParams(9, 1, 0.0, 0.0, 0, 0, 0, 1, 0)
    assert L.hsa_select(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 4, NULL, 0, NULL) == 6


def test_select_noalloc_validation(B):
    """The allocation-free selection checks its arguments like hsa_select and
    refuses, before any launch, a problem whose workspace exceeds its static
    array."""
    L = B.lib()
    p = B.make_params("thresh_global", tau=0.25, budget_ratio=0.3)
    assert L.hsa_select_noalloc(FAKE, 512, 1024, ctypes.byref(p), FAKE, FAKE, 1024, NULL) == 4
    assert b"static scratch" in L.hsa_last_error()
    assert L.hsa_select_noalloc(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 3, NULL) == 2     # max_kv != nb
    assert L.hsa_select_noalloc(NULL, 2, 4, ctypes.byref(p), FAKE, FAKE, 4, NULL) == 1
    p = B.make_params("thresh_global", tau=4.0, budget_ratio=0.3)
    assert L.hsa_select_noalloc(FAKE, 2, 4, ctypes.byref(p), FAKE, FAKE, 4, NULL) == 6
    assert b"hsa_select_noalloc" in L.hsa_last_error()


def test_radial_select_validation_and_width(B):
    L = B.lib()
    p = B.make_params("radial", frames=61, tiles_per_frame=13, lam=0.125)
    width = L.hsa_select_list_width(12, 793, ctypes.byref(p))
    assert width == 169
    assert L.hsa_select(NULL, 12, 793, ctypes.byref(p), FAKE, FAKE, width - 1, NULL, 0, NULL) == 2
    assert L.hsa_select(NULL, 12, 792, ctypes.byref(p), FAKE, FAKE, width, NULL, 0, NULL) == 2
    p = B.make_params("radial", frames=61, tiles_per_frame=13, lam=1.5)
    assert L.hsa_select(NULL, 12, 793, ctypes.byref(p), FAKE, FAKE, 793, NULL, 0, NULL) == 6
    assert L.hsa_select_list_width(12, 793, ctypes.byref(p)) == 0
    p = B.make_params("radial_dyn", frames=61, tiles_per_frame=13, lam=0.1, delta=1.0)
    assert L.hsa_select_list_width(12, 793, ctypes.byref(p)) == 793
    assert L.hsa_select(NULL, 12, 793, ctypes.byref(p), FAKE, FAKE, 793, NULL, 0, NULL) == 1   # S
    assert L.hsa_select(FAKE, 12, 793, ctypes.byref(p), FAKE, FAKE, 792, NULL, 0, NULL) == 2   # max_kv
    p = B.make_params("radial_dyn", frames=61, tiles_per_frame=13, lam=0.1, delta=-1.0)
    assert L.hsa_select(FAKE, 12, 793, ctypes.byref(p), FAKE, FAKE, 793, NULL, 0, NULL) == 6
    p = B.make_params("topk", k=7)
    assert L.hsa_select_list_width(2, 16, ctypes.byref(p)) == 7


def test_attn_and_unperm_validation(B):
    L = B.lib()
    a = [FAKE] * 8
    assert L.hsa_attn(NULL, *a[1:4], NULL, *a[5:8], NULL, 4, 0, 2, 4, 64, 64, 1, 0.125, NULL) == 1
    assert L.hsa_attn(*a[:4], NULL, *a[5:8], NULL, 4, 0, 2, 4, 96, 64, 1, 0.125, NULL) == 4      # B
    assert L.hsa_attn(*a[:4], NULL, *a[5:8], NULL, 4, 4, 2, 4, 64, 64, 1, 0.125, NULL) == 6      # kv_shared
    assert L.hsa_attn(*a[:4], NULL, *a[5:8], NULL, 4, 0, 2, 4, 64, 64, 1, float("nan"), NULL) == 6
    assert L.hsa_attn(*a[:4], NULL, *a[5:8], ctypes.c_void_p(0x10002), 4, 0, 2, 4, 64, 64, 1, 0.125,
                      NULL) == 6                                                                 # order alignment
    assert L.hsa_attn_order(NULL, 2, 4, 4, FAKE, NULL) == 1
    assert L.hsa_attn_order(FAKE, 0, 4, 4, FAKE, NULL) == 2
    assert L.hsa_attn_order(FAKE, 2, 4, 4096, FAKE, NULL) == 4                                   # max_kv
    assert L.hsa_attn_order(FAKE, 1 << 16, 1 << 16, 4, FAKE, NULL) == 4                          # G*nb
    # hsa_attn_tokens(q, k, v, o, q_stride, kv_stride, o_stride, lse, perm, N, blk_len, kv_idx,
    #                 kv_cnt, order, max_kv, kv_shared, nh, nb, B, D, dtype, scale, stream)
    def tok(q_stride=128, kv_stride=0, o_stride=128, perm=FAKE, N=200, B_=64, order=NULL, nh=2):
        return L.hsa_attn_tokens(FAKE, FAKE, FAKE, FAKE, q_stride, kv_stride, o_stride, NULL, perm, N,
                                 FAKE, FAKE, FAKE, order, 4, 0, nh, 4, B_, 64, 1, 0.125, NULL)
    assert tok(perm=NULL) == 1
    assert tok(N=0) == 2 and tok(N=257) == 2                                                     # N vs nb*B
    assert tok(q_stride=100) == 2 and tok(o_stride=64) == 2 and tok(kv_stride=64) == 2           # stride < nh*D
    assert tok(q_stride=132) == 6 and tok(o_stride=132) == 6 and tok(kv_stride=132) == 6         # 16-byte rows
    assert tok(kv_stride=-8) == 6                                                                # negative
    assert tok(B_=96) == 4
    assert tok(order=ctypes.c_void_p(0x10002)) == 6
    # gathered K/V rows use 32-bit byte offsets: a 4 GiB token-major span is refused
    assert L.hsa_attn_tokens(FAKE, FAKE, FAKE, FAKE, 1 << 14, 1 << 14, 1 << 14, NULL, FAKE, 1 << 17,
                             FAKE, FAKE, FAKE, NULL, 4, 0, 128, 1024, 128, 128, 1, 0.125, NULL) == 4
    # ... and their offsets use 24-bit factors: more than 2^24 tokens, or rows of 16 MiB, are refused
    assert L.hsa_attn_tokens(FAKE, FAKE, FAKE, FAKE, 128, 128, 128, NULL, FAKE, (1 << 24) + 64,
                             FAKE, FAKE, FAKE, NULL, 4, 0, 2, (1 << 18) + 1, 64, 64, 1, 0.125, NULL) == 4
    assert L.hsa_attn_tokens(FAKE, FAKE, FAKE, FAKE, 128, 1 << 23, 128, NULL, FAKE, 200,
                             FAKE, FAKE, FAKE, NULL, 4, 0, 2, 4, 64, 64, 1, 0.125, NULL) == 4
    assert b"2^24" in L.hsa_last_error()
    assert L.hsa_unperm(FAKE, FAKE, FAKE, 10, 8, 2, 64, 128, 1, NULL) == 2
    assert L.hsa_unperm(FAKE, NULL, FAKE, 10, 16, 2, 64, 128, 1, NULL) == 1


def test_header_is_plain_c_and_links(tmp_path):
    """A C99 program includes the header, links the library and calls it."""
    exe = tmp_path / "abi_smoke"
    src = os.path.join(ROOT, "tests", "c", "abi_smoke.c")
    build = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                            "-o", str(exe), "-L", os.path.dirname(LIB), "-lhsa",
                            "-Wl,-rpath," + os.path.dirname(LIB)], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.startswith("ok 4 workspace too small")
