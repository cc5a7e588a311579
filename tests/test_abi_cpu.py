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
    # deferred expert weight gradients: 2..16 slots, bf16 only, not with the recomputation rule
    (dict(max_microbatches=1), B.MOE_OK), (dict(max_microbatches=16), B.MOE_OK),
    (dict(max_microbatches=17), B.MOE_ERR_ARG), (dict(max_microbatches=-1), B.MOE_ERR_ARG),
    (dict(max_microbatches=4, dtype="f32"), B.MOE_ERR_ARG),
    (dict(max_microbatches=4, memory_rules=B.MOE_MEM_RECOMPUTE), B.MOE_ERR_ARG),
    (dict(max_microbatches=16, max_tokens=1 << 24, top_k=4), B.MOE_ERR_SHAPE),
    # memory rules: the two known bits alone or together; any other bit is refused
    (dict(memory_rules=B.MOE_MEM_GUARDS), B.MOE_OK),
    (dict(memory_rules=B.MOE_MEM_GUARDS | B.MOE_MEM_RECOMPUTE), B.MOE_OK),
    (dict(memory_rules=B.MOE_MEM_GUARDS, max_microbatches=4), B.MOE_OK),
    (dict(memory_rules=0x4), B.MOE_ERR_ARG),
])
def test_config_validation(kw, expect):
    base = dict(d_model=64, d_ff=128, n_experts=4, top_k=2, max_tokens=256, dtype="bf16")
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
    damaged = ctypes.c_int32(7)
    assert lib.moe_step_check_guards(None, ctypes.byref(damaged)) == B.MOE_ERR_ARG and damaged.value == 0
    assert lib.moe_step_check_guards(None, None) == B.MOE_ERR_ARG
    lib.moe_step_destroy(None)
    assert isinstance(B.moe_step_last_error(None), str)


def _layer_without_handle(dtype):
    # the tensor checks of MoeLayerStep.run, on a layer object with no device
    # handle: its "device" is the CPU, so tensors can be made here
    import torch
    from moe_step_megakernel_amd.layer import MoeLayerStep
    layer = object.__new__(MoeLayerStep)
    layer.cfg = B.make_config(16, 24, 4, 2, 64, dtype)
    layer.dtype = dtype
    layer.dev = torch.device("cpu")
    layer.handle = None
    layer.trace_words = lambda: 100
    return layer


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_checks_tensors_before_any_pointer_is_passed(dtype):
    import torch
    layer = _layer_without_handle(dtype)
    act = torch.bfloat16 if dtype == "bf16" else torch.float32
    other = torch.float32 if dtype == "bf16" else torch.bfloat16
    x = torch.zeros(10, 16, dtype=act)
    ok = dict(dx=torch.zeros(10, 16), router_bias=torch.zeros(4),
              debug={"router_logits": torch.zeros(10, 4), "topk_idx": torch.zeros(10, 2, dtype=torch.int32),
                     "topk_gate": torch.zeros(10, 2), "expert_counts": torch.zeros(4, dtype=torch.int32),
                     "route_perm": torch.zeros(20, dtype=torch.int32)},
              trace=torch.zeros(100, dtype=torch.int64))
    layer._check_tensors(10, x, x, **ok)
    layer._check_tensors(0, None, None, None, None, {}, None)
    bad = [
        dict(x=x.to(other)),                                   # activation dtype of the other mode
        dict(target=torch.zeros(10, 8, dtype=act)),            # wrong width
        dict(x=torch.zeros(16, 10, dtype=act).t()),            # not contiguous
        dict(target=None),                                     # x without target
        dict(dx=torch.zeros(10, 16, dtype=torch.float64)),
        dict(dx=torch.zeros(9, 16)),
        dict(router_bias=torch.zeros(5)),
        dict(debug={"topk_idx": torch.zeros(10, 2, dtype=torch.int64)}),
        dict(debug={"route_perm": torch.zeros(10, dtype=torch.int32)}),
        dict(debug={"logits": torch.zeros(10, 4)}),            # unknown name
        dict(trace=torch.zeros(99, dtype=torch.int64)),        # too short
    ]
    for change in bad:
        args = dict(x=x, target=x, **ok)
        args.update(change)
        with pytest.raises((TypeError, ValueError)):
            layer._check_tensors(10, args["x"], args["target"], args["dx"], args["router_bias"], args["debug"],
                                 args["trace"])


def test_static_entry_refuses_guard_zones_before_hip():
    import torch
    cfg = B.make_config(64, 128, 4, 2, 256, memory_rules=B.MOE_MEM_GUARDS)
    io = B.make_io(stats=torch.zeros(4))   # checked for NULL only; refused before any HIP call
    lib = B.load_library()
    assert lib.moe_step_run_static(ctypes.byref(cfg), ctypes.byref(io), 16, 16, 1, 0, None) == B.MOE_ERR_ARG
    assert "MOE_MEM_GUARDS" in B.moe_step_last_error(None)
