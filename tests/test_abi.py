"""The C ABI without a GPU: the library loads, exports every symbol that
include/awq_mi355x.h declares, and rejects bad arguments on the host before
anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from post_bit_weight_awq_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq_mi355x.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(awq_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libawq_mi355x.so is not built (run post_bit_weight_awq_amd/build.py)")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_default_config_and_version(lib):
    cfg = _lib.AwqConfig()
    lib.awq_default_config(ctypes.byref(cfg))
    assert (cfg.w_bit, cfg.group_size, cfg.n_grid, cfg.zero_point) == (4, 128, 20, 1)
    assert cfg.sal_floor == pytest.approx(1e-4, rel=1e-6)
    assert b"gfx950" in lib.awq_version()


def _cfg(lib, **kw):
    cfg = _lib.AwqConfig()
    lib.awq_default_config(ctypes.byref(cfg))
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg


FAKE = ctypes.c_void_p(0x1000)      # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x1004)


@pytest.mark.parametrize("kw,code", [
    (dict(w_bit=2), _lib.AWQ_ERR_UNSUPPORTED),
    (dict(w_bit=8), _lib.AWQ_ERR_UNSUPPORTED),
    (dict(group_size=16), _lib.AWQ_ERR_UNSUPPORTED),
    (dict(group_size=256), _lib.AWQ_ERR_UNSUPPORTED),
    (dict(zero_point=2), _lib.AWQ_ERR_UNSUPPORTED),
    (dict(n_grid=0), _lib.AWQ_ERR_INVALID_ARG),
    (dict(n_grid=65), _lib.AWQ_ERR_INVALID_ARG),
    (dict(sal_floor=0.0), _lib.AWQ_ERR_INVALID_ARG),
    (dict(sal_floor=float("nan")), _lib.AWQ_ERR_INVALID_ARG),
])
def test_search_rejects_bad_config(lib, kw, code):
    cfg = _cfg(lib, **kw)
    rc = lib.awq_search_layer(FAKE, FAKE, FAKE, 128, 512, 512, ctypes.byref(cfg), FAKE, FAKE,
                              FAKE, FAKE, 1 << 40, None)
    assert rc == code
    assert lib.awq_last_error()
    rc = lib.awq_pack(FAKE, FAKE, 512, 512, ctypes.byref(cfg), FAKE, FAKE, FAKE, None)
    assert rc == code


@pytest.mark.parametrize("n,k,o", [(0, 512, 512), (128, 500, 512), (128, 512, 0),
                                   (128, 0, 512), ((1 << 24) + 1, 512, 512),
                                   (128, 1 << 21, 8)])
def test_search_rejects_bad_shapes(lib, n, k, o):
    cfg = _cfg(lib)
    rc = lib.awq_search_layer(FAKE, FAKE, FAKE, n, k, o, ctypes.byref(cfg), FAKE, FAKE, FAKE,
                              FAKE, 1 << 40, None)
    assert rc == _lib.AWQ_ERR_INVALID_ARG
    assert lib.awq_search_workspace_size(n, k, o, ctypes.byref(cfg)) == 0


def test_search_rejects_null_and_misaligned(lib):
    cfg = _cfg(lib)
    args = [FAKE, FAKE, FAKE, 128, 512, 512, ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, 1 << 40,
            None]
    for pos in (0, 1, 2, 7, 8, 9, 10):
        a = list(args)
        a[pos] = None
        assert lib.awq_search_layer(*a) == _lib.AWQ_ERR_INVALID_ARG, pos
    for pos in (0, 1, 2, 7, 9, 10):
        a = list(args)
        a[pos] = MISALIGNED
        assert lib.awq_search_layer(*a) == _lib.AWQ_ERR_INVALID_ARG, pos
        assert b"aligned" in lib.awq_last_error()


def test_search_workspace_too_small(lib):
    cfg = _cfg(lib)
    need = lib.awq_search_workspace_size(128, 512, 512, ctypes.byref(cfg))
    assert need > 0
    rc = lib.awq_search_layer(FAKE, FAKE, FAKE, 128, 512, 512, ctypes.byref(cfg), FAKE, FAKE,
                              FAKE, FAKE, need - 1, None)
    assert rc == _lib.AWQ_ERR_WORKSPACE


@pytest.mark.parametrize("n", [500, 1024, 1025, 4096])
def test_search_plan_layout(lib, n):
    # up to 1024 tokens (four 256-token tiles): the fused grid kernel and its
    # parameter table; from 1025 (five tiles): the contraction path and its
    # weight error
    cfg = _cfg(lib)
    plan = _lib.AwqSearchPlan()
    assert lib.awq_search_plan_query(n, 4096, 1000, ctypes.byref(cfg), ctypes.byref(plan)) == 0
    assert plan.n_token_tiles == -(-n // plan.tile_tokens)
    assert plan.n_out_tiles == -(-1000 // plan.tile_out)
    contraction = n >= 1025
    assert (plan.tile_tokens, plan.tile_out) == ((256, 256) if contraction else
                                                 (plan.tile_tokens, 128))
    regions = sorted([
        (plan.partials_offset, 16 * 20 * plan.n_token_tiles * plan.n_out_tiles),
        (plan.scales_offset, 4 * 20 * 4096)])
    for (a, la), (b, _) in zip(regions, regions[1:]):
        assert a + la <= b
    assert regions[-1][0] + regions[-1][1] <= plan.workspace_bytes
    for off in (plan.partials_offset, plan.scales_offset):
        assert off % 256 == 0
    # the scale tables and either the per-group parameters or the fp16 weight
    # error of every grid point dominate; there is no N x OUT buffer
    payload = 2 * 20 * 1000 * 4096 if contraction else 16 * 20 * 1000 * (4096 // 128)
    assert payload < plan.workspace_bytes
    assert plan.workspace_bytes < payload + 2 * 4 * 20 * 4096 + 16 * 20 * 64 + 4096


def test_stats_validation(lib):
    assert lib.awq_act_stats_workspace_size(0, 512) == 0
    assert lib.awq_act_stats_workspace_size(10, 12) == 0
    need = lib.awq_act_stats_workspace_size(10, 512)
    assert need >= 8 * 512
    assert lib.awq_act_stats(None, 10, 512, FAKE, FAKE, need, None) == _lib.AWQ_ERR_INVALID_ARG
    assert lib.awq_act_stats(FAKE, 10, 512, FAKE, FAKE, need - 8, None) == _lib.AWQ_ERR_WORKSPACE
    assert lib.awq_act_stats(FAKE, 10, 512, MISALIGNED, FAKE, need, None) == _lib.AWQ_ERR_INVALID_ARG


def test_stats_noalloc_validation(lib):
    # rejected on the host before the device is touched: bad pointers, bad
    # shapes, and partial sums beyond the fixed scratch (2 row chunks x 2^20
    # columns x 8 bytes = 16 MiB > 8 MiB)
    f = lib.awq_act_stats_noalloc
    assert f(None, 10, 512, FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, 10, 512, None, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, 10, 512, MISALIGNED, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, 0, 512, FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, 10, 12, FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, 8193, 1 << 20, FAKE, None) == _lib.AWQ_ERR_WORKSPACE
    assert b"scratch" in lib.awq_last_error()


def test_pack_validation(lib):
    cfg = _cfg(lib)
    assert lib.awq_pack(FAKE, FAKE, 100, 4, ctypes.byref(cfg), FAKE, FAKE, FAKE, None) \
        == _lib.AWQ_ERR_INVALID_ARG
    assert lib.awq_pack(FAKE, FAKE, 128, 4, ctypes.byref(cfg), FAKE, None, FAKE, None) \
        == _lib.AWQ_ERR_INVALID_ARG
    assert lib.awq_pack(FAKE, FAKE, 128, 4, ctypes.byref(cfg), FAKE, ctypes.c_void_p(0x1001),
                        FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert lib.awq_pack(FAKE, FAKE, 128, 4, None, FAKE, FAKE, FAKE, None) \
        == _lib.AWQ_ERR_INVALID_ARG


def test_python_binding_rejects_cpu_tensors():
    import torch
    import post_bit_weight_awq_amd as awq
    X = torch.zeros(4, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        awq.awq_act_stats(X, out=torch.empty(128), workspace=torch.empty(4096, dtype=torch.uint8))


@pytest.mark.parametrize("n,k", [(1, 8), (63, 512), (64, 4096), (512, 4096), (4096, 13824),
                                 (9000, 64), ((1 << 20) + 3, 1024)])
def test_stats_workspace_bounds(lib, n, k):
    need = lib.awq_act_stats_workspace_size(n, k)
    assert need % 8 == 0
    assert 8 * k <= need <= 8 * k * (1 + n // 64)


def test_w4a16_validation(lib):
    args = [FAKE, 4, 256, 32, FAKE, FAKE, FAKE, FAKE, None]
    for pos, bad in ((1, 0), (1, (1 << 20) + 1), (2, 200), (2, 0), (3, 0)):
        a = list(args)
        a[pos] = bad
        assert lib.awq_w4a16_matmul(*a) == _lib.AWQ_ERR_INVALID_ARG, (pos, bad)
    for pos in (0, 4, 5, 6, 7):
        a = list(args)
        a[pos] = None
        assert lib.awq_w4a16_matmul(*a) == _lib.AWQ_ERR_INVALID_ARG, pos
    for pos, ptr in ((0, MISALIGNED), (4, MISALIGNED), (5, ctypes.c_void_p(0x1001)),
                     (7, ctypes.c_void_p(0x1002))):
        a = list(args)
        a[pos] = ptr
        assert lib.awq_w4a16_matmul(*a) == _lib.AWQ_ERR_INVALID_ARG, pos
        assert lib.awq_last_error()


def test_fold_validation(lib):
    f = lib.awq_fold_inverse_scale
    assert f(None, FAKE, 4, 1, FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 0, 1, FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 4, 0, FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(0x1001), FAKE, 4, 1, FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, ctypes.c_void_p(0x1002), 4, 1, ctypes.c_void_p(0x2000), None) \
        == _lib.AWQ_ERR_INVALID_ARG
    # dst overlapping src by part of the array
    assert f(ctypes.c_void_p(0x1000), FAKE, 4, 8, ctypes.c_void_p(0x1010), None) \
        == _lib.AWQ_ERR_INVALID_ARG
    assert b"overlap" in lib.awq_last_error()


def test_select_top_validation(lib):
    f = lib.awq_select_top_channels
    assert f(None, 8, 1, FAKE, None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, 0, 0, ctypes.c_void_p(0x2000), None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, 8, 9, ctypes.c_void_p(0x2000), None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(FAKE, 8, -1, ctypes.c_void_p(0x2000), None) == _lib.AWQ_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(0x1002), 8, 1, ctypes.c_void_p(0x2000), None) \
        == _lib.AWQ_ERR_INVALID_ARG
    assert f(ctypes.c_void_p(0x1000), 8, 1, ctypes.c_void_p(0x1004), None) \
        == _lib.AWQ_ERR_INVALID_ARG


def test_bench_cpu_baseline_fields():
    # the oracle baseline of the benchmark line, on the small configuration:
    # the rate over a bounded sample, the threads it used and what it sampled
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_for_cpu", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    r = bench.cpu_baseline(1, 0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert r["host"]["affinity_cores"] >= 1 and r["host"]["blas_threads"] >= 1
    assert [x["layer"] for x in r["per_layer"]] == ["linear"]
    assert set(r["seconds"]) == {"stats", "search", "pack"}
    assert "single_linear_in512_out512_tok128" in r["sample"]


def test_bench_refuses_more_than_one_gpu():
    # the path runs on one GPU: a multi-GPU request exits with a message
    # before any device work
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_grid_profiles_match_the_grid_source():
    # every committed summary of the grid kernel names the digest of the code
    # it was taken on; a kernel edit without new counters shows up here (and
    # the benchmark then reports its traffic as null)
    import glob
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_for_digest", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    digest = bench.source_digest()
    paths = sorted(glob.glob(os.path.join(root, "profiles", "*.md")))
    named = 0
    for p in paths:
        txt = open(p).read()
        for m in re.finditer(r"(?:source digest[^:]*:\s*|source=)([0-9a-f]{16})", txt):
            named += 1
            assert m.group(1) == digest, os.path.basename(p)
    assert named >= 3
    assert bench.traffic_from_profiles("llama13b_block_h5120_mlp13824_tok4096") is not None
