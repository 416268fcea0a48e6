"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/sa.h declares, and rejects invalid arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")
LIB = os.path.join(ROOT, "indexer_routed_sparse_amd", "libsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsa.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ["sa_indexer_scores", "sa_topk_select", "sa_sparse_mla_fwd", "sa_block_sparse_gqa_fwd",
              "sa_status_string", "sa_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for n in _declared():
        assert hasattr(lib, n), n


def test_debug_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(os.path.join(ROOT, "indexer_routed_sparse_amd", "libsa_debug.so"))
    for n in _declared():
        assert hasattr(lib, n), n
    lib.sa_abi_version.restype = ctypes.c_int
    assert lib.sa_abi_version() == 3


def test_version_and_status_strings():
    import indexer_routed_sparse_amd as sa
    assert sa.abi_version() == 3
    for code in range(8):
        assert sa.status_string(code).startswith("SA_")
    assert "unknown" in sa.status_string(99)


def _lib():
    import indexer_routed_sparse_amd as sa
    return sa.lib


P = ctypes.c_void_p
FAKE = P(0x10000)          # aligned, never dereferenced: every call below fails validation
MIS = P(0x10004)


@pytest.mark.parametrize("args,code", [
    # (q, kv, idx, dtype, T, S, H, d_qk, d_v, topk, scale, out, lse) -> status
    ((FAKE, FAKE, FAKE, 7, 4, 4, 16, 576, 512, 8, 1.0, FAKE, None), 3),   # dtype
    ((FAKE, FAKE, FAKE, 1, 4, 4, 16, 100, 512, 8, 1.0, FAKE, None), 5),   # d_qk
    ((FAKE, FAKE, FAKE, 1, 4, 4, 16, 576, 256, 8, 1.0, FAKE, None), 5),   # d_v
    ((FAKE, FAKE, FAKE, 1, 4, 4, 256, 576, 512, 8, 1.0, FAKE, None), 5),  # H > 128
    ((FAKE, FAKE, FAKE, 1, 4, 4, 24, 576, 512, 8, 1.0, FAKE, None), 5),   # H % 16
    ((FAKE, FAKE, FAKE, 1, 4, 0, 16, 576, 512, 8, 1.0, FAKE, None), 2),   # S
    ((FAKE, FAKE, FAKE, 1, 4, 1 << 21, 16, 576, 512, 8, 1.0, FAKE, None), 5),  # kv > 2 GiB
    ((FAKE, FAKE, FAKE, 1, 4, 4, 16, 576, 512, 0, 1.0, FAKE, None), 2),   # topk
    ((None, FAKE, FAKE, 1, 4, 4, 16, 576, 512, 8, 1.0, FAKE, None), 1),   # null q
    ((FAKE, FAKE, FAKE, 1, 4, 4, 16, 576, 512, 8, 1.0, None, None), 1),   # null out
    ((MIS, FAKE, FAKE, 1, 4, 4, 16, 576, 512, 8, 1.0, FAKE, None), 4),    # misaligned q
])
def test_sparse_mla_rejects(args, code):
    lib = _lib()
    a = list(args)
    a.insert(11, None)                                  # sink
    assert lib.sa_sparse_mla_fwd(*a, None) == code


def test_sparse_mla_empty_is_ok():
    assert _lib().sa_sparse_mla_fwd(None, None, None, 1, 0, 4, 16, 576, 512, 8, 1.0, None, None, None, None) == 0


@pytest.mark.parametrize("args,code", [
    # (vals, cand, ld, T, cu, nseq, maxlen, B, topk, force, out_idx, out_val)
    ((FAKE, None, 6, 4, None, 0, 0, 1, 2, 0, FAKE, None), 2),        # ld % 4
    ((FAKE, None, 4, 8, None, 0, 0, 1, 2, 0, FAKE, None), 2),        # ld < row width
    ((FAKE, None, 8, 8, None, 0, 0, 1, 0, 0, FAKE, None), 2),        # topk 0
    ((FAKE, None, 8, 8, None, 0, 0, 1, 2, 1, FAKE, None), 5),        # force own in token mode
    ((FAKE, FAKE, 8, 8, None, 0, 0, 1, 2, 1, FAKE, None), 5),        # force own with candidates
    ((FAKE, None, 131072, 131072, None, 0, 0, 1, 2, 0, FAKE, None), 5),  # row too wide
    ((None, None, 8, 8, None, 0, 0, 1, 2, 0, FAKE, None), 1),        # null vals
    ((MIS, None, 8, 8, None, 0, 0, 1, 2, 0, FAKE, None), 4),         # misaligned
    ((FAKE, None, 8, 8, FAKE, 0, 8, 1, 2, 0, FAKE, None), 2),        # cu without sequences
])
def test_topk_select_rejects(args, code):
    assert _lib().sa_topk_select(*args, None) == code


@pytest.mark.parametrize("args,code", [
    # (q, k, w, dtype, T, cu, nseq, maxlen, H_I, D_I, B, scores, ld, topk, force, idx, val)
    ((FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 3, 128, 1, FAKE, 8, 0, 0, None, None), 5),   # H_I
    ((FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 96, 1, FAKE, 8, 0, 0, None, None), 5),   # D_I
    ((FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 128, 48, FAKE, 8, 0, 0, None, None), 5), # B
    ((FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 128, 3, FAKE, 8, 0, 0, None, None), 5),  # B odd
    ((FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 128, 1, FAKE, 4, 0, 0, None, None), 2),  # ld small
    ((FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 128, 1, None, 0, 4096, 0, FAKE, None), 5),  # topk
    ((FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 128, 1, FAKE, 8, 4, 0, FAKE, None), 2),  # both modes
    ((FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 128, 1, None, 0, 4, 0, None, None), 1),  # no out_idx
    ((FAKE, FAKE, FAKE, 9, 8, None, 0, 0, 64, 128, 1, FAKE, 8, 0, 0, None, None), 3),  # dtype
])
def test_indexer_rejects(args, code):
    assert _lib().sa_indexer_scores(*args, None, 0, None) == code


def _ws_bytes(dtype, T, maxlen, H_I, D_I, B, topk):
    lib = _lib()
    lib.sa_indexer_workspace_bytes.restype = ctypes.c_size_t
    return lib.sa_indexer_workspace_bytes(dtype, T, maxlen, H_I, D_I, B, topk)


def test_indexer_workspace_sizes():
    # token mode: two-pass route only for bf16, 64 heads, fused selection
    long = _ws_bytes(1, 32768, 32768, 64, 128, 1, 2048)
    assert 32768 * 2048 * 8 < long < 32768 * 8192 * 8          # a few thousand entries per row
    assert long % 4 == 0
    assert _ws_bytes(1, 32768, 32768, 64, 128, 1, 0) == 0          # dense mode
    assert _ws_bytes(1, 32768, 32768, 16, 128, 1, 2048) == 0       # generic kernel
    assert _ws_bytes(0, 32768, 32768, 64, 128, 1, 2048) == 0       # fp32
    assert _ws_bytes(1, 0, 1, 64, 128, 1, 16) == 0                 # nothing to do
    # block mode: key ranges split in runs of 32 tiles of 64 keys, at most 4, each run's
    # top-k ([T, splits, topk] keys and ids), [T, splits] counts, [T] own values
    assert _ws_bytes(1, 2048, 2048, 16, 128, 64, 16) == 0          # 32 tiles: one pass
    assert _ws_bytes(1, 4096, 4096, 16, 128, 64, 16) == 4096 * (2 * 16 * 8 + 2 * 4 + 4)
    assert _ws_bytes(1, 8192, 8192, 16, 128, 64, 16) == 8192 * (4 * 16 * 8 + 4 * 4 + 4)
    assert _ws_bytes(0, 32768, 32768, 64, 128, 64, 16) == 32768 * (4 * 16 * 8 + 4 * 4 + 4)   # fp32 too
    assert _ws_bytes(1, 8192, 8192, 16, 128, 64, 0) == 0           # dense block scores
    # rows never wider than the row: short sequences take the whole row
    assert _ws_bytes(1, 1000, 1000, 64, 128, 1, 2048) == 1000 * 1024 * 8 + 1000 * 4
    # packed sequences size by the widest one
    assert _ws_bytes(1, 65536, 16384, 64, 128, 1, 2048) < _ws_bytes(1, 65536, 65536, 64, 128, 1, 2048)


def test_indexer_rejects_small_workspace():
    need = _ws_bytes(1, 8, 8, 64, 128, 1, 4)
    assert need > 0
    args = (FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 128, 1, None, 0, 4, 0, FAKE, None)
    assert _lib().sa_indexer_scores(*args, FAKE, need - 1, None) == 7     # SA_ERR_WORKSPACE
    assert _lib().sa_indexer_scores(*args, MIS, need, None) == 4          # misaligned workspace


@pytest.mark.parametrize("args,code", [
    # (q, k, v, blk, dtype, T, cu, nseq, maxlen, Hq, Hkv, D, Dv, B, nblk, scale, out, lse)
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 30, 4, 128, 128, 64, 16, 1.0, FAKE, None), 2),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 64, 2, 128, 128, 64, 16, 1.0, FAKE, None), 5),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 32, 4, 96, 96, 64, 16, 1.0, FAKE, None), 5),
    ((FAKE, FAKE, FAKE, FAKE, 1, 8, None, 0, 0, 32, 4, 128, 128, 40, 16, 1.0, FAKE, None), 5),
    ((FAKE, FAKE, FAKE, None, 1, 8, None, 0, 0, 32, 4, 128, 128, 64, 16, 1.0, FAKE, None), 1),
])
def test_block_gqa_rejects(args, code):
    assert _lib().sa_block_sparse_gqa_fwd(*args, None) == code
