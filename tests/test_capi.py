"""C ABI contract, checked on the CPU: the library loads, exports every symbol
the header declares, and rejects bad arguments before launching anything
(only argument errors are exercised here, so no kernel runs)."""
import ctypes
import os
import re

import pytest

import long_context_indexer_block_amd as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(H.LIB_PATH), reason="libhisa.so not built")

FAKE = ctypes.c_void_p(0x10000)     # aligned, never dereferenced: every call below fails validation
NULL = ctypes.c_void_p(0)
S = H.Strides


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hisa_status_t|size_t|const char\*|int)\s+(\w+)\(",
                                 txt, flags=re.M)))


def test_exports_match_header():
    names = _declared()
    assert len(names) == 21
    lib = ctypes.CDLL(H.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(H.EXPORTS) == names
    assert H.lib().hisa_abi_version() == 3


def _err():
    return H.lib().hisa_last_error().decode()


def test_block_summary_validation():
    L = H.lib()
    st = L.hisa_block_summary(NULL, S(0, 64, 0), 1, 128, 64, 64, NULL, FAKE, NULL, NULL)
    assert st == 1 and "kidx" in _err()
    st = L.hisa_block_summary(FAKE, S(0, 64, 0), 1, 128, 96, 64, NULL, FAKE, NULL, NULL)
    assert st == 3 and "d=96" in _err()
    st = L.hisa_block_summary(FAKE, S(0, 64, 0), 1, 128, 64, 48, NULL, FAKE, NULL, NULL)
    assert st == 3 and "B=48" in _err()
    st = L.hisa_block_summary(FAKE, S(0, 60, 0), 1, 128, 64, 64, NULL, FAKE, NULL, NULL)
    assert st == 2 and "strides" in _err()
    st = L.hisa_block_summary(ctypes.c_void_p(0x10002), S(0, 64, 0), 1, 128, 64, 64, NULL, FAKE,
                              NULL, NULL)
    assert st == 2 and "aligned" in _err()
    st = L.hisa_block_summary(FAKE, S(0, 64, 0), 1, 128, 64, 64, NULL, NULL, NULL, NULL)
    assert st == 1


def test_select_and_token_validation():
    L = H.lib()
    assert L.hisa_select_blocks(FAKE, FAKE, 1, 4, 8, 64, 1, FAKE, NULL) == 3      # m < 2
    assert "m=1" in _err()
    # token select: workspace too small, missing, k too large, m*B too large
    args = [FAKE, S(0, 64, 0), FAKE, S(0, 64, 0), FAKE, FAKE, 1, 16, 1024, 64, 64, 4, 8, FAKE,
            NULL]
    need = L.hisa_token_select_workspace_bytes(1, 16, 1024, 64, 4, 8)
    assert need > 0
    assert L.hisa_token_select(*args, NULL, need, NULL) == 5
    assert L.hisa_token_select(*args, FAKE, need - 1, NULL) == 5 and "needs" in _err()
    bad = list(args)
    bad[12] = 20000
    assert L.hisa_token_select(*bad, FAKE, need, NULL) == 3
    bad = list(args)
    bad[11] = 512
    bad[10] = 64
    assert L.hisa_token_select(*bad, FAKE, 1 << 40, NULL) == 3 and "m*B" in _err()


def test_attention_validation():
    L = H.lib()
    s = S(0, 128, 128)
    base = [FAKE, s, FAKE, s, FAKE, s, 1, 4, 64, 6, 4, 128, 128, FAKE, 8, 0.1, FAKE, s, NULL,
            NULL, 0, NULL]
    assert L.sparse_attn_fwd(*base) == 2 and "multiple" in _err()     # Hq % Hkv
    b2 = list(base)
    b2[9], b2[10] = 128, 1
    assert L.sparse_attn_fwd(*b2) == 3                               # group > 64
    b3 = list(base)
    b3[9], b3[10], b3[11], b3[12] = 4, 4, 96, 96
    assert L.sparse_attn_fwd(*b3) == 3 and "(96, 96)" in _err()
    b4 = list(base)
    b4[9], b4[10], b4[15] = 4, 4, -1.0
    assert L.sparse_attn_fwd(*b4) == 2 and "scale" in _err()
    b5 = list(base)
    b5[0] = NULL
    assert L.sparse_attn_fwd(*b5) == 1


def test_attention_out_checks():
    # the kernels store whole 16-byte pieces of out: a misaligned base or a
    # stride that is not a multiple of 8 elements is rejected before launch
    L = H.lib()
    s = S(0, 128 * 16, 128)
    args = [FAKE, s, FAKE, S(0, 128, 128), FAKE, S(0, 128, 128), 1, 4, 64, 16, 1, 128, 128,
            FAKE, 8, 0.1]
    assert L.sparse_attn_fwd(*args, ctypes.c_void_p(0x10008), s, NULL, NULL, 0, NULL) == 2
    assert "out" in _err() and "aligned" in _err()
    assert L.sparse_attn_fwd(*args, FAKE, S(0, 128 * 16, 132), NULL, NULL, 0, NULL) == 2
    assert "out" in _err() and "strides" in _err()
    assert L.sparse_attn_fwd(*args, FAKE, S(0, -2048, 128), NULL, NULL, 0, NULL) == 2
    assert "out" in _err()
    mla = [FAKE, S(0, 576 * 64, 576), FAKE, S(0, 576, 576), FAKE, S(0, 576, 576), 1, 4, 64, 64,
           1, 576, 512, FAKE, 8, 0.1]
    assert L.sparse_attn_fwd(*mla, ctypes.c_void_p(0x10004), S(0, 512 * 64, 512), NULL, NULL,
                             0, NULL) == 2 and "out" in _err()


def test_gather_probe_validation():
    L = H.lib()
    args = [FAKE, 1152, 1152, 1024, FAKE, 16, 2048, 4, 2, 0, NULL]
    a = list(args)
    a[0] = NULL
    assert L.hisa_gather_probe(*a) == 1
    a = list(args)
    a[2] = 512                                                       # row width
    assert L.hisa_gather_probe(*a) == 3 and "row_bytes" in _err()
    a = list(args)
    a[7] = 6                                                         # waves
    assert L.hisa_gather_probe(*a) == 3
    a = list(args)
    a[8] = 5                                                         # depth
    assert L.hisa_gather_probe(*a) == 3
    a = list(args)
    a[6] = 4097                                                      # topk
    assert L.hisa_gather_probe(*a) == 3
    a = list(args)
    a[9] = -1                                                        # rotation period
    assert L.hisa_gather_probe(*a) == 2
    a = list(args)
    a[1] = 1144                                                      # stride below the row
    assert L.hisa_gather_probe(*a) == 2 and "row_stride" in _err()
    a = list(args)
    a[0] = ctypes.c_void_p(0x10004)
    assert L.hisa_gather_probe(*a) == 2 and "aligned" in _err()


NO_DEVICE = not os.path.exists("/dev/kfd")


@pytest.mark.skipif(not NO_DEVICE, reason="launches with placeholder pointers: only on a host "
                                          "without a GPU, where the launch itself must fail")
def test_launch_error_is_hip_status():
    # every check passes, so the call reaches the HIP launch, which fails for
    # want of a device: HISA_ERR_HIP with HIP's own text, prefixed by the entry
    L = H.lib()
    st = L.hisa_gather_probe(FAKE, 1152, 1152, 1024, FAKE, 16, 2048, 4, 2, 0, NULL)
    assert st == 4
    msg = _err()
    assert msg.startswith("hisa_gather_probe: ") and len(msg) > len("hisa_gather_probe: ")
    s = S(0, 128, 128)
    st = L.sparse_attn_fwd(FAKE, s, FAKE, s, FAKE, s, 1, 4, 64, 1, 1, 128, 128, FAKE, 8, 0.1,
                           FAKE, s, NULL, NULL, 0, NULL)
    assert st == 4 and _err().startswith("sparse_attn_fwd: ")
    # a later failing check replaces the text
    assert L.hisa_gather_probe(NULL, 1152, 1152, 1024, FAKE, 16, 2048, 4, 2, 0, NULL) == 1
    assert "required" in _err()


def test_token_select_noalloc_limits():
    # the allocation-free form: same checks as the workspace form, and shapes
    # whose scratch exceeds the fixed array are rejected before any HIP call
    L = H.lib()
    args = [FAKE, S(0, 128, 0), FAKE, S(0, 128, 0), FAKE, FAKE, 1, 16384, 16384, 128, 128, 32,
            2048, FAKE, NULL, NULL]
    assert L.hisa_token_select_workspace_bytes(1, 16384, 16384, 128, 32, 2048) > 64 << 20
    assert L.hisa_token_select_noalloc(*args) == 3 and "scratch" in _err()
    a = list(args)
    a[13] = NULL
    assert L.hisa_token_select_noalloc(*a) == 1
    a = list(args)
    a[11] = 1                                                        # m < 2
    assert L.hisa_token_select_noalloc(*a) == 3
    a = list(args)
    a[13] = ctypes.c_void_p(0x10004)                                 # token_idx alignment
    assert L.hisa_token_select_noalloc(*a) == 2


def test_attention_workspace():
    L = H.lib()
    # few (query, kv head) pairs with long lists split (decode: 64 x 16 heads
    # over 2048 tokens); many pairs, short lists and the MLA shape do not
    need = L.sparse_attn_fwd_workspace_bytes(64, 1, 16, 1, 128, 128, 2048)
    assert need > 0 and need % 256 == 0
    assert L.sparse_attn_fwd_workspace_bytes(1, 16384, 16, 1, 128, 128, 2048) == 0
    assert L.sparse_attn_fwd_workspace_bytes(1, 1, 16, 1, 128, 128, 32) == 0
    assert L.sparse_attn_fwd_workspace_bytes(1, 4, 64, 1, 576, 512, 2048) == 0
    assert L.sparse_attn_fwd_workspace_bytes(1, 4, 6, 4, 128, 128, 2048) == 0   # Hq % Hkv
    s = S(0, 128 * 16, 128)
    args = [FAKE, s, FAKE, S(0, 128, 128), FAKE, S(0, 128, 128), 64, 1, 4096, 16, 1, 128, 128,
            FAKE, 2048, 0.1, FAKE, s, NULL]
    assert L.sparse_attn_fwd(*args, FAKE, need - 1, NULL) == 5 and "needs" in _err()
    assert L.sparse_attn_fwd(*args, ctypes.c_void_p(0x10010), need, NULL) == 5
    assert "aligned" in _err()


def test_hils_validation():
    L = H.lib()
    s = S(0, 64, 64)
    args = [FAKE, s, FAKE, s, FAKE, s, FAKE, FAKE, 1, 4096, 16, 64, 64, 64, 32, 0.125, 0.125,
            FAKE, s, NULL, 0, NULL]
    a = list(args)
    a[13] = 63                                                       # n_rows != ceil(L/C)
    assert L.hils_two_level_attn_fwd(*a) == 2
    a = list(args)
    a[14] = 65                                                       # m > 64
    assert L.hils_two_level_attn_fwd(*a) == 3
    a = list(args)
    a[11] = 32                                                       # D unsupported
    assert L.hils_two_level_attn_fwd(*a) == 3
    # few (sequence, head) pairs split their chunks; many do not
    need = L.hils_two_level_attn_fwd_workspace_bytes(1, 16, 64, 32)
    assert need > 0 and need % 256 == 0
    assert L.hils_two_level_attn_fwd_workspace_bytes(64, 16, 64, 32) == 0
    a = list(args)
    a[19], a[20] = FAKE, need - 1                                    # too small
    assert L.hils_two_level_attn_fwd(*a) == 5 and "needs" in _err()


def test_route_validation():
    L = H.lib()
    s = S(0, 64, 0)
    args = [FAKE, s, FAKE, 1, 4096, FAKE, 64, 64, 64, 32, FAKE, NULL, 0, NULL]
    a = list(args)
    a[6], a[9] = 1027, 131                       # too many blocks for LDS, m too large to stream
    assert L.hisa_route_blocks(*a) == 3 and "hisa_block_score" in _err()
    a = list(args)
    a[6] = 65538                                                     # too many to stream
    assert L.hisa_route_blocks(*a) == 3
    a = list(args)
    a[9] = 1                                                         # m < 2
    assert L.hisa_route_blocks(*a) == 3
    a = list(args)
    a[8] = 96                                                        # B unsupported
    assert L.hisa_route_blocks(*a) == 3
    a = list(args)
    a[10] = NULL                                                     # no output
    assert L.hisa_route_blocks(*a) == 1


def test_route_workspace():
    L = H.lib()
    # few queries over many blocks split their blocks over workgroups
    need = L.hisa_route_blocks_workspace_bytes(64, 1, 1024, 64)      # 128K decode batch
    assert need > 0 and need % 256 == 0
    assert need >= 64 * 4 * 62 * 8
    assert L.hisa_route_blocks_workspace_bytes(16, 1, 16384, 32) > 0  # 1M two-level decode
    assert L.hisa_route_blocks_workspace_bytes(1, 4096, 1024, 64) == 0  # many queries
    assert L.hisa_route_blocks_workspace_bytes(64, 1, 1024, 67) == 0    # m - 2 > 64
    assert L.hisa_route_blocks_workspace_bytes(1, 1, 65537, 64) == 0    # too many survivors
    assert L.hisa_route_blocks_workspace_bytes(0, 1, 1024, 64) == 0
    s = S(0, 128, 0)
    args = [FAKE, s, FAKE, 64, 1, FAKE, 1024, 128, 128, 64, FAKE, FAKE, need, NULL]
    a = list(args)
    a[12] = need - 1                                                 # too small
    assert L.hisa_route_blocks(*a) == 5 and "needs" in _err()
    a = list(args)
    a[11] = ctypes.c_void_p(0x10010)                                 # not 256-byte aligned
    assert L.hisa_route_blocks(*a) == 5 and "aligned" in _err()


def test_hils_prefill_validation():
    L = H.lib()
    s = S(0, 1024, 64)
    args = [FAKE, s, FAKE, s, FAKE, s, FAKE, FAKE, FAKE, FAKE, 1, 4096, 4096, 16, 64, 64, 64, 32,
            0.125, 0.125, FAKE, s, NULL, 0, NULL]
    a = list(args)
    a[9] = NULL                                                      # q_pos missing
    assert L.hils_two_level_prefill_fwd(*a) == 1
    a = list(args)
    a[8] = NULL                                                      # no proj: plain means, valid
    a[16] = 63                                                       # but n_rows != ceil(L/C)
    assert L.hils_two_level_prefill_fwd(*a) == 2 and "n_rows" in _err()
    a = list(args)
    a[11] = 0                                                        # nq < 1
    assert L.hils_two_level_prefill_fwd(*a) == 2
    a = list(args)
    a[17] = 1                                                        # m < 2
    assert L.hils_two_level_prefill_fwd(*a) == 3
    a = list(args)
    a[14] = 96                                                       # D unsupported
    assert L.hils_two_level_prefill_fwd(*a) == 3
    a = list(args)
    a[10], a[13] = 4097, 16                                          # batch*H > 65535
    assert L.hils_two_level_prefill_fwd(*a) == 3 and "65535" in _err()
    a = list(args)
    a[2] = ctypes.c_void_p(0x10002)                                  # k not 16-byte aligned
    assert L.hils_two_level_prefill_fwd(*a) == 2
    a = list(args)
    a[1] = S(0, 1024, 4)                                             # q head stride not 8k
    assert L.hils_two_level_prefill_fwd(*a) == 2
    a = list(args)
    a[21] = S(0, 1020, 64)                                           # out token stride not 8k
    assert L.hils_two_level_prefill_fwd(*a) == 2 and "out" in _err()
    # the bucketed path's scratch: per-entry partials dominate
    need = L.hils_two_level_prefill_fwd_workspace_bytes(1, 4096, 4096, 16, 64, 64, 32)
    assert need >= 16 * 4096 * 32 * 64 * 2 and need % 256 == 0
    assert L.hils_two_level_prefill_fwd_workspace_bytes(1, 4096, 4096, 16, 96, 64, 32) == 0
    a = list(args)
    a[22], a[23] = FAKE, need - 1                                    # too small
    assert L.hils_two_level_prefill_fwd(*a) == 5 and "needs" in _err()
    a = list(args)
    a[22], a[23] = ctypes.c_void_p(0x10010), need                    # not 256-byte aligned
    assert L.hils_two_level_prefill_fwd(*a) == 5 and "aligned" in _err()


def test_missing_library_raises(monkeypatch):
    monkeypatch.setattr(H, "_lib", None)
    monkeypatch.setattr(H, "LIB_PATH", "/nonexistent/libhisa.so")
    with pytest.raises(H.HisaError):
        H.lib()


def test_auto_plan():
    """The runtime policy (HISA explainer 1.3 item 3; 3.2 item 2): the flat
    indexer below 8192 keys, m = max(64, L // 2000), clamped to m*B <= 16384."""
    for L, B, hier, m in [(1, 128, False, 64), (8191, 128, False, 64), (8192, 128, True, 64),
                          (16384, 64, True, 64), (65536, 128, True, 64), (131072, 128, True, 65),
                          (200000, 128, True, 100), (1048576, 64, True, 256),
                          (1048576, 128, True, 128), (1048576, 256, True, 64)]:
        assert H.hisa_auto_plan(L, B) == (hier, m), (L, B)
    L = H.lib()
    x, y = ctypes.c_int(0), ctypes.c_int(0)
    assert L.hisa_auto_plan(0, 128, ctypes.byref(x), ctypes.byref(y)) == 2
    assert L.hisa_auto_plan(4096, 96, ctypes.byref(x), ctypes.byref(y)) == 3
    assert L.hisa_auto_plan(4096, 128, None, ctypes.byref(y)) == 1
