"""C-ABI library: loads, exports every function include/fp2.h declares, and
rejects malformed arguments on the host before any HIP call (these calls
never reach a kernel, so they run without a GPU)."""
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
lib = pytest.importorskip("block_sparse_long_blocks_amd")
import torch  # noqa: E402


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fp2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp2_[a-z_]+)\s*\(", src)))


def test_library_is_the_one_requested():
    """The in-tree libfp2.so, or the build a test run asked for (the sanitized host build)."""
    want = os.environ.get("FP2_TEST_LIBRARY") or os.path.join(ROOT, "block_sparse_long_blocks_amd", "libfp2.so")
    assert os.path.realpath(lib.library_path()) == os.path.realpath(want)


def test_exports_every_declared_function():
    import ctypes
    names = declared_functions()
    assert len(names) >= 7
    so = ctypes.CDLL(lib.library_path())
    for n in names:
        assert hasattr(so, n), n


def _batch(seqlens, nq, block=128, kv_block=0):
    return lib.Batch(block, seqlens, nq, device="cpu", kv_block=kv_block)


def _kv(hkv=2, d=128, page=128, pages=4, dtype=torch.bfloat16, maxp=4):
    kp = torch.zeros((pages, page, hkv, d), dtype=dtype)
    return lib.KVCache(kp, kp.clone(), torch.zeros((1, maxp), dtype=torch.int32))


def _q(total, hq=4, d=128, dtype=torch.bfloat16):
    return lib.Queries(torch.zeros((max(total, 1), hq, d), dtype=dtype))


def _expect(code, fn, *args, match=None, **kw):
    with pytest.raises(lib.Fp2Error) as e:
        fn(*args, **kw)
    assert e.value.status == code, str(e.value)
    if match:
        assert re.search(match, str(e.value)), str(e.value)


def test_sizes_and_counts():
    b = _batch([1000, 256], [1000, 128])
    # seq0: 8 q-blocks, diag 0..7 -> 36; seq1: prefix 128 -> P/B = 1, 1 q-block -> 2
    assert lib.fp2_plan_max_nnz(b, 3) == 3 * (36 + 2)
    assert lib.fp2_plan_workspace_bytes(b, 3) > 0
    # d = 128, B = 128: bf16 kbar rows plus a 128 x 128 bf16 V^T tile per KV block and head
    # (e4m3: V dequantized, the same parts, no copy of K: about the size of the e4m3 K and V);
    # and the float32 partials of split rows: up to 2 * extra slots (extra = min(256, causal
    # tiles / 4, rounded up) = 29 here) of 8 waves x 4224 floats per 256 packed query rows
    tiles = 3 * (8 + 2) * 128 * 128 * 2
    parts = 2 * 29 * 2 * 8 * 4224 * 4  # 12 q heads / 3 kv heads: 512 packed rows = 2 slices
    assert lib.fp2_run_workspace_bytes(b, 12, 3, 128, lib.FP2_BF16) >= tiles + 3 * (8 + 2) * 128 * 2 + parts
    assert lib.fp2_run_workspace_bytes(b, 12, 3, 128, lib.FP2_FP8_E4M3) == \
        lib.fp2_run_workspace_bytes(b, 12, 3, 128, lib.FP2_BF16)
    assert lib.fp2_run_workspace_bytes(b, 12, 3, 128, lib.FP2_FP8_E4M3) < 2 * tiles + parts
    assert lib.fp2_run_workspace_bytes(b, 24, 3, 128, lib.FP2_BF16) >= \
        lib.fp2_run_workspace_bytes(b, 12, 3, 128, lib.FP2_BF16) + parts
    assert lib.fp2_run_workspace_bytes(b, 2, 3, 128, lib.FP2_BF16) == 0
    # other head sizes: bf16 kbar + fp16 vbar copies only
    assert lib.fp2_run_workspace_bytes(b, 12, 3, 64, lib.FP2_BF16) < tiles
    assert lib.fp2_run_workspace_bytes(b, 12, 3, 64, lib.FP2_FP8_E4M3) >= 2 * 3 * (8 + 2) * 64 * 2


def test_stage1_sizes_and_checks():
    """fp2_stage1: its workspace is the plan workspace plus float32 pooled query means
    [Hkv, total_qblocks, d] (256-byte aligned) plus 256 bytes for the selection pass's work
    counter; its checks are those of the two calls it fuses."""
    b = _batch([1000, 256], [1000, 128])
    plan = lib.fp2_plan_workspace_bytes(b, 3)
    qbar = 3 * (8 + 1) * 128 * 4
    assert lib.fp2_stage1_workspace_bytes(b, 3, 128) == plan + ((qbar + 255) & ~255) + 256
    f32 = torch.zeros(16)
    i32 = torch.zeros(64, dtype=torch.int32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    bb = _batch([256], [256])
    kv = _kv()
    _expect(lib.FP2_ERR_CAPACITY, lib.fp2_stage1, bb, _q(256), kv, 1.0, f32, f32, i32, i32, i32, ws[:8],
            match="stage-1 workspace")
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_stage1, bb, lib.Queries(torch.zeros((256, 4, 128), dtype=torch.uint8),
            f32), kv, 1.0, f32, f32, i32, i32, i32, ws, match="dtypes differ")
    _expect(lib.FP2_ERR_INVALID, lib.fp2_stage1, bb, _q(256), kv, math.nan, f32, f32, i32, i32, i32, ws,
            match="NaN")
    _expect(lib.FP2_ERR_CAPACITY, lib.fp2_stage1, bb, _q(256), kv, 1.0, f32, f32, i32, i32[:5], i32, ws)
    _expect(lib.FP2_ERR_INVALID, lib.fp2_stage1, bb, _q(256), kv, 1.0, None, f32, i32, i32, i32, ws, match="NULL")
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_stage1, _batch([256], [256], 32), _q(256), kv, 1.0, f32, f32, i32,
            i32, i32, ws, match="block")


def test_decoupled_blocks_sizes_and_counts():
    """128-token query blocks over 64-token KV blocks: the causal count is that of the blocks
    holding a visible key (counted here from positions); workspace layouts per path."""
    seqlens, nq = [1000, 300, 256], [1000, 172, 128]
    b = _batch(seqlens, nq, 128, 64)
    want = 0
    for T, n in zip(seqlens, nq):
        P = T - n
        for i in range(-(-n // 128)):
            last = P + min(128 * (i + 1), n) - 1          # the query block's last position
            want += len([J for J in range(-(-T // 64)) if 64 * J <= last])
    assert lib.fp2_plan_max_nnz(b, 2) == 2 * want
    # same batch with one block size: the same positions at 128-token granularity
    assert lib.fp2_plan_max_nnz(_batch(seqlens, nq), 2) < 2 * want
    assert lib.fp2_plan_max_nnz(_batch(seqlens, nq, 128, 128), 2) == lib.fp2_plan_max_nnz(_batch(seqlens, nq), 2)
    # d = 128: the DMA kernel's layout with a 128 d x 64 key V^T half tile per block and head
    # (e4m3: the same parts); d = 64 runs the register-staged kernel: kbar / vbar copies only
    nkb = sum(-(-T // 64) for T in seqlens)
    assert lib.fp2_run_workspace_bytes(b, 8, 2, 128, lib.FP2_BF16) >= 2 * nkb * 128 * 64 * 2
    assert lib.fp2_run_workspace_bytes(b, 8, 2, 128, lib.FP2_FP8_E4M3) == \
        lib.fp2_run_workspace_bytes(b, 8, 2, 128, lib.FP2_BF16)
    assert lib.fp2_run_workspace_bytes(b, 8, 2, 64, lib.FP2_BF16) < 2 * 2 * nkb * 64 * 2 + 1024
    # one block-stats cache row per 64-token block a page holds
    assert lib.fp2_block_stats_cache_rows(_batch([256], [256], 128, 64), _kv(page=128)) == 8
    assert lib.fp2_block_stats_cache_rows(_batch([256], [256], 128, 64), _kv(page=32, pages=8, maxp=8)) == 8
    f32 = torch.zeros(16)
    for B, KB in ((128, 32), (64, 128), (64, 32), (128, 96)):
        _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_block_stats, _batch([256], [256], B, KB), _kv(), f32, f32,
                match="kv_block")
    # e4m3 scales are per page: the page must be the 64-token KV block
    kv8 = lib.KVCache(torch.zeros((4, 128, 2, 128), dtype=torch.uint8),
                      torch.zeros((4, 128, 2, 128), dtype=torch.uint8),
                      torch.zeros((1, 4), dtype=torch.int32), f32, f32)
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_block_stats, _batch([256], [256], 128, 64), kv8, f32, f32,
            match="KV block")
    # the prefix is still a multiple of the query block
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_block_stats, _batch([320], [256], 128, 64), _kv(), f32, f32,
            match="prefix")


def test_sequence_length_limits():
    """2^21 keys (16,384 blocks of 128) is the largest sequence accepted; one block more is
    rejected on the host (the kept-block bitmask and the plan's score row live in LDS)."""
    assert lib.fp2_plan_max_nnz(_batch([1 << 21], [256]), 1) == 16383 + 16384  # diagonals 16382, 16383
    assert lib.fp2_plan_max_nnz(_batch([(1 << 21) + 128], [256]), 1) == -1
    # 64-token KV blocks under 128-token query blocks: 16,384 of them is 2^20 keys
    assert lib.fp2_plan_max_nnz(_batch([1 << 20], [256], 128, 64), 1) == 16382 + 16384  # runs 16380-1, 16382-3
    assert lib.fp2_plan_max_nnz(_batch([(1 << 20) + 64], [320], 128, 64), 1) == -1


def test_int32_csr_limit():
    """row_ptr, col_idx and nnz are int32: two 2^21-token sequences with 8 KV heads have
    2 * 16384 * 16385 / 2 * 8 = 2,147,614,720 causal pairs > 2^31 - 1, so a dense plan
    would wrap; the host rejects the batch before any launch.  One sequence fits."""
    f32 = torch.zeros(16)
    i32 = torch.zeros(16, dtype=torch.int32)
    ws = torch.zeros(16, dtype=torch.uint8)
    big = _batch([1 << 21, 1 << 21], [1 << 21, 1 << 21])
    assert lib.fp2_plan_max_nnz(big, 8) == 2 * 16384 * 16385 // 2 * 8 > (1 << 31) - 1
    q = lib.Queries(torch.zeros((1, 32, 128), dtype=torch.bfloat16))  # pointers only: nothing is launched
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_plan_mask, big, q, 8, f32, math.inf, i32, i32, i32, ws,
            match="2\\^31")
    kv = _kv(hkv=8, maxp=16384)
    out = torch.zeros(8)
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_prefill_run, big, q, kv, i32, i32, f32, f32, False, out, ws,
            match="2\\^31")
    # one such sequence is 1,073,807,360 pairs: past the index check, stopped by the capacity check
    one = _batch([1 << 21], [1 << 21])
    _expect(lib.FP2_ERR_CAPACITY, lib.fp2_plan_mask, one, q, 8, f32, math.inf, i32, i32, i32, ws)


def test_noalloc_plan_rejects_batches_beyond_its_scratch():
    """fp2_plan_mask_noalloc's workspace is a fixed 8 MiB device array: a batch whose plan
    workspace is larger (one sequence with 16,384 KV blocks, so 512 bitmask words a row, plus
    4,096 one-block sequences: 4,097 query blocks x 8 KV heads = 32,776 rows, 67 MB) is refused
    on the host before anything is launched; the same batch passes the other checks."""
    seqlens = [1 << 21] + [128] * 4096
    nq = [128] + [128] * 4096
    b = _batch(seqlens, nq)
    need = lib.fp2_plan_workspace_bytes(b, 8)
    assert need > 8 << 20
    f32 = torch.zeros(16)
    i32 = torch.zeros(16, dtype=torch.int32)
    q = lib.Queries(torch.zeros((1, 32, 128), dtype=torch.bfloat16))  # pointers only: nothing is launched
    cols = torch.zeros(lib.fp2_plan_max_nnz(b, 8), dtype=torch.int32)
    _expect(lib.FP2_ERR_CAPACITY, lib.fp2_plan_mask_noalloc, b, q, 8, f32, 1.0, i32, cols, i32,
            match="allocation-free")
    # a too-small col_capacity is still reported first, as fp2_plan_mask does
    _expect(lib.FP2_ERR_CAPACITY, lib.fp2_plan_mask_noalloc, b, q, 8, f32, 1.0, i32, i32, i32,
            match="col_capacity")


def test_block_stats_cache_rows_and_checks():
    """The paged block-stats cache: one row per KV block a page holds; page sizes that do not
    divide B (or the reverse) are unsupported; bad arguments are rejected before any launch."""
    b = _batch([256], [256])
    assert lib.fp2_block_stats_cache_rows(b, _kv(page=64)) == 4          # a block spans 2 pages: keyed by its first
    assert lib.fp2_block_stats_cache_rows(b, _kv(page=128)) == 4
    assert lib.fp2_block_stats_cache_rows(b, _kv(page=256, pages=2)) == 4  # 2 blocks per page
    assert lib.fp2_block_stats_cache_rows(b, _kv(page=96)) == 0
    f32 = torch.zeros(16)
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_block_stats_cached, b, _kv(page=96), f32, f32, True, match="page_size")
    _expect(lib.FP2_ERR_INVALID, lib.fp2_block_stats_cached, b, _kv(), None, f32, False, match="NULL")
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_gather_block_stats, b, _kv(page=96), f32, f32, f32, f32,
            match="page_size")
    _expect(lib.FP2_ERR_INVALID, lib.fp2_gather_block_stats, b, _kv(), f32, f32, None, f32, match="NULL")


def test_validation_rejects_before_launch():
    f32 = torch.zeros(16)
    i32 = torch.zeros(16, dtype=torch.int32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    b = _batch([256], [256])
    # block size
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_block_stats, _batch([256], [256], 32), _kv(), f32, f32,
            match="block")
    # prefix not a multiple of block
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_block_stats, _batch([300], [200]), _kv(), f32, f32,
            match="prefix")
    # more queries than keys
    _expect(lib.FP2_ERR_INVALID, lib.fp2_block_stats, _batch([100], [200]), _kv(), f32, f32)
    # head_dim
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_block_stats, b, _kv(d=96), f32, f32, match="head_dim")
    # fp8 with page_size != block
    kv8 = lib.KVCache(torch.zeros((4, 64, 2, 128), dtype=torch.uint8),
                      torch.zeros((4, 64, 2, 128), dtype=torch.uint8),
                      torch.zeros((1, 8), dtype=torch.int32), f32, f32)
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_block_stats, b, kv8, f32, f32, match="page_size")
    # too few pages in the table
    _expect(lib.FP2_ERR_INVALID, lib.fp2_block_stats, _batch([1024], [1024]), _kv(maxp=4), f32, f32,
            match="max_pages_per_seq")
    # GQA: Hq not a multiple of Hkv
    _expect(lib.FP2_ERR_INVALID, lib.fp2_plan_mask, b, _q(256, hq=3), 2, f32, 1.0, i32, i32, i32, ws)
    # tau NaN
    _expect(lib.FP2_ERR_INVALID, lib.fp2_plan_mask, b, _q(256), 2, f32, math.nan, i32, i32, i32, ws,
            match="NaN")
    # col capacity below the causal count: 2 q-blocks -> 3 pairs x 2 heads = 6
    _expect(lib.FP2_ERR_CAPACITY, lib.fp2_plan_mask, b, _q(256), 2, f32, 1.0, i32, i32[:5], i32, ws)
    # plan workspace too small
    _expect(lib.FP2_ERR_CAPACITY, lib.fp2_plan_mask, b, _q(256), 2, f32, 1.0, i32, i32, i32, ws[:8])
    # fp8 queries without scales
    _expect(lib.FP2_ERR_INVALID, lib.fp2_plan_mask, b, lib.Queries(torch.zeros((256, 4, 128), dtype=torch.uint8)),
            2, f32, 1.0, i32, i32, i32, ws, match="q_scale")
    # dtype mismatch between q and kv
    out = torch.zeros(8)
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_prefill_run, b,
            lib.Queries(torch.zeros((256, 4, 128), dtype=torch.uint8), f32), _kv(), i32, i32, f32, f32, True,
            out, ws)
    # run workspace too small for the correction
    _expect(lib.FP2_ERR_CAPACITY, lib.fp2_prefill_run, b, _q(256), _kv(), i32, i32, f32, f32, True, out, ws[:4])
    # bad softmax scale
    _expect(lib.FP2_ERR_INVALID, lib.fp2_prefill_run, b, _q(256), _kv(), i32, i32, f32, f32, False, out, ws,
            softmax_scale=-1.0)
    # group too wide for the pooling pass
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_plan_mask, b, _q(256, hq=64), 2, f32, 1.0, i32, i32, i32, ws)


def test_release_build_has_no_bounds_word():
    """Without FP2_DEBUG_BOUNDS the library trusts page ids and the CSR, and says so instead of
    reporting a word it does not keep (no HIP call is made)."""
    _expect(lib.FP2_ERR_UNSUPPORTED, lib.fp2_debug_bounds_word, match="FP2_DEBUG_BOUNDS")


def test_bounds_build_is_built():
    """build() also builds libfp2_bounds.so (FP2_DEBUG_BOUNDS) beside libfp2.so; it exports the same
    functions."""
    import ctypes
    path = os.path.join(ROOT, "block_sparse_long_blocks_amd", "libfp2_bounds.so")
    assert os.path.exists(path), "build it: python block_sparse_long_blocks_amd/build.py --debug-bounds"
    so = ctypes.CDLL(path)
    for n in declared_functions():
        assert hasattr(so, n), n


def test_no_fallback_without_library(tmp_path, monkeypatch):
    """The binding refuses to import when libfp2.so is absent (no CPU path)."""
    import importlib.util
    src = os.path.join(ROOT, "block_sparse_long_blocks_amd", "_binding.py")
    dst = tmp_path / "_binding.py"
    dst.write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("binding_copy", str(dst))
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="not built"):
        spec.loader.exec_module(mod)


def test_build_entry_builds_before_importing_the_package(tmp_path):
    """__graft_entry__.build() must work where libfp2.so is not built yet: it may not import the
    package (whose import loads the library) before the build step has run.  The build step is a
    stand-in here that copies the library built in this tree into the copy."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "block_sparse_long_blocks_amd"
    shutil.copytree(os.path.join(ROOT, "block_sparse_long_blocks_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    shutil.copy(os.path.join(ROOT, "__graft_entry__.py"), tmp_path)
    (pkg / "build.py").write_text(
        "import os, shutil\n"
        f"SRC = {lib.library_path()!r}\n"
        "def build(debug=False, bounds=False):\n"
        "    name = 'libfp2_bounds.so' if bounds else 'libfp2.so'\n"
        "    dst = os.path.join(os.path.dirname(os.path.abspath(__file__)), name)\n"
        "    shutil.copy(SRC, dst)\n"
        "    return dst\n")
    assert not (pkg / "libfp2.so").exists()
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "built" in r.stdout
