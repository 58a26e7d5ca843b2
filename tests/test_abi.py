"""The C ABI: both builds load and export every function include/skv.h declares."""
import os
import re

import pytest

from lora_shared_kv_amd import skv as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "skv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(skv_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("skv_append_base", "skv_append_lowrank", "skv_attn_prefill", "skv_attn_decode",
                     "skv_crop", "skv_create", "skv_destroy"):
        assert required in names
    assert set(names) == set(B.EXPORTS), set(names) ^ set(B.EXPORTS)


@pytest.mark.parametrize("kind", ["gpu", "host"])
def test_library_exports_every_declared_symbol(kind):
    path = B.library_path(kind)
    assert os.path.exists(path), f"{path} not built"
    lib = B.load_library(kind)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_gpu_library_links_hip_and_not_the_null_backend():
    import subprocess
    path = B.library_path("gpu")
    syms = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    assert "skv_attn_decode" in syms
    deps = subprocess.run(["ldd", path], capture_output=True, text=True).stdout
    assert "libamdhip64" in deps
    # the null device backend is compiled only into the host build
    allsyms = subprocess.run(["nm", "-C", path], capture_output=True, text=True).stdout
    assert "decode_split_kernel" in allsyms


def test_arena_bytes_and_config_validation():
    cfg = dict(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, hidden=1024, rank=8,
               n_agents=2, mode=0, page_size=64, max_pages=16)
    n = B.skv_arena_bytes(cfg, "host")
    assert n > 0
    pools = 2 * 2 * 16 * 2 * 64 * 128 * 2            # K and V^T
    assert n >= pools
    bad = dict(cfg, head_dim=96)
    assert B.skv_arena_bytes(bad, "host") == 0
    with pytest.raises(B.SkvError) as e:
        B.skv_create(bad, (1 << 20, 1 << 30), None, "host")
    assert e.value.code == "ARG"
    with pytest.raises(B.SkvError) as e:
        B.skv_create(cfg, (1 << 20, n - 1), None, "host")   # arena too small
    assert e.value.code == "ARG"


def test_gpu_build_rejects_page_sizes_it_does_not_handle():
    # the device check runs before any GPU call, so this works without a GPU
    cfg = dict(n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=64, hidden=64, rank=4,
               n_agents=2, mode=0, page_size=32, max_pages=8)
    with pytest.raises(B.SkvError) as e:
        B.skv_create(cfg, (1 << 20, 1 << 40), 0, "gpu")
    assert e.value.code == "UNSUPPORTED"


def test_bench_refuses_more_than_one_gpu():
    # the bench measures one GPU; asking for several must fail before any GPU work
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_bench_kernel_names_follow_the_library_choices():
    # the template arguments bench.py reports must be the ones the library
    # instantiates (decode split blocks, front-end tiles)
    import bench
    kernels = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                "lora_shared_kv_amd", "csrc", "kernels.hip")).read()
    assert bench.split_kernel_name(128, 16, 1, 8) == "decode_split_kernel<128,1,1>"
    assert bench.project_kernel_name(32, 8, 128, 4) == "project_split_kernel<128>"
    assert bench.project_kernel_name(32, 8, 128, 384) == "project_wide_kernel<128,4,3>"
    assert bench.project_kernel_name(32, 8, 128, 512) == "project_wide_kernel<128,4,4>"
    assert bench.project_kernel_name(32, 8, 128, 1024) == "project_tall_kernel<128>"
    assert bench.project_kernel_name(32, 8, 128, 4096) == "project_tall_kernel<128>"
    assert "launch_project_split<D>(g, p)" in kernels
    for nh in (3, 4):
        assert f"launch_project_wide<D, {nh}>(g, p)" in kernels
    assert "launch_project_tall<D>(g, p)" in kernels
