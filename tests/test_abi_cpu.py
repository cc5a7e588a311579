"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/moe_step.h, sizes parameters and validates configurations
and arguments before touching HIP."""
import ctypes
import os
import re

import pytest

from moe_step_megakernel_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe_step.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_step_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    names = _declared_functions()
    assert len(names) >= 8, names
    for name in names:
        assert hasattr(lib, name), f"missing export {name}"
        assert hasattr(B, name), f"binding lacks {name}"


def test_config_struct_size_matches_library():
    cfg = B.make_config(768, 1536, 16, 2, 2048)
    assert B.moe_step_check_config(cfg) == B.MOE_OK     # the library checks struct_size == sizeof
    cfg.struct_size -= 4
    assert B.moe_step_check_config(cfg) == B.MOE_ERR_ARG


@pytest.mark.parametrize("d,f,E,k,expect", [(768, 1536, 16, 2, 37761024), (64, 128, 4, 2, 65792),
                                             (1024, 512, 64, 8, 67174400)])
def test_param_count(d, f, E, k, expect):
    assert B.moe_step_param_count(B.make_config(d, f, E, k, 16)) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(d_model=0), B.MOE_ERR_ARG), (dict(top_k=5, n_experts=4), B.MOE_ERR_ARG),
    (dict(d_model=12), B.MOE_ERR_SHAPE), (dict(d_ff=100), B.MOE_ERR_SHAPE),
    (dict(n_experts=65), B.MOE_ERR_SHAPE), (dict(top_k=9, n_experts=16), B.MOE_ERR_SHAPE),
    (dict(max_tokens=0), B.MOE_ERR_ARG), (dict(beta1=1.0), B.MOE_ERR_ARG), (dict(wg_per_cu=3), B.MOE_ERR_ARG),
    (dict(max_tokens=(1 << 24) + 1), B.MOE_ERR_SHAPE),
])
def test_config_validation(kw, expect):
    base = dict(d_model=64, d_ff=128, n_experts=4, top_k=2, max_tokens=256)
    base.update(kw)
    cfg = B.make_config(**base)
    assert B.moe_step_check_config(cfg) == expect


def test_abi_version_checked():
    cfg = B.make_config(64, 128, 4, 2, 256)
    cfg.abi_version = 99
    assert B.moe_step_check_config(cfg) == B.MOE_ERR_ARG


def test_create_rejects_bad_config_before_hip():
    cfg = B.make_config(64, 100, 4, 2, 256)
    with pytest.raises(B.MoeStepError) as ei:
        B.moe_step_create(cfg)
    assert ei.value.status == B.MOE_ERR_SHAPE
    assert "multiples of 8" in B.moe_step_last_error(None)


def test_create_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(B.MoeStepError) as ei:
        B.moe_step_create(B.make_config(64, 128, 4, 2, 256))
    assert ei.value.status in (B.MOE_ERR_HIP, B.MOE_ERR_DEVICE)


def test_null_handle_calls_are_safe():
    lib = B.load_library()
    assert lib.moe_step_run(None, None, 0, 1, 1, 0, None) == B.MOE_ERR_ARG
    assert lib.moe_step_run_groups(None, None, 0, 1, 1, 1, 0, None) == B.MOE_ERR_ARG
    assert lib.moe_step_status(None) == B.MOE_ERR_ARG
    assert lib.moe_step_trace_words(None) == 0
    assert lib.moe_step_grid_size(None) == 0
    assert lib.moe_step_arena_bytes(None) == 0
    lib.moe_step_destroy(None)
    assert isinstance(B.moe_step_last_error(None), str)
