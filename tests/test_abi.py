"""The C-ABI library loads and exports every symbol include/moe.h declares, and
its host-side validation rejects bad arguments before launching anything.
CPU only: no call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from mixture_experts_sparse_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    from mixture_experts_sparse_amd import load
    return load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_five_steps():
    names = declared_functions()
    for n in ["moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    lib = ctypes.CDLL(L.LIB_PATH)
    names = declared_functions()
    assert names, "no declarations parsed"
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(L.EXPORTED) == names


def test_struct_layout_matches_header(L):
    assert ctypes.sizeof(L.moe_config) == 17 * 4  # static_assert'ed in moe_api.hip too
    assert ctypes.sizeof(L.moe_expert_weights) == 12 * 8
    assert ctypes.sizeof(L.moe_routing_out) == 4 * 8
    assert ctypes.sizeof(L.moe_kernel_time) == 64


def test_status_strings(L):
    lib = L.lib()
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(3) == b"workspace too small"
    assert lib.moe_version() >= 100


def _cfg(L, **kw):
    base = W.WORKLOADS["mixtral_bf16"]
    return L.make_config(base.replace(**kw))


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), 1), (dict(E=257), 1), (dict(k=9), 1), (dict(k=0), 1), (dict(T=-1), 1),
    (dict(d=100), 2), (dict(F=100), 2), (dict(tau=0.0), 1), (dict(tau=-1.0), 1),
    (dict(score=5), 1), (dict(bias_mode=7), 1), (dict(n_shared=2), 1),
    (dict(act_dtype=W.DT_F32), 2), (dict(w_dtype=W.DT_F32), 2), (dict(w_dtype=9), 1),
    (dict(score=W.SCORE_SIGMOID, tau=0.5), 2), (dict(score=W.SCORE_SIGMOID, bias_mode=W.BIAS_LOGIT), 2),
    (dict(capacity_factor=float("inf")), 1), (dict(renormalize=3), 1),
    (dict(reroute_depth=-1), 1), (dict(reroute_depth=9, E=64), 1), (dict(reroute_depth=7), 1),
    (dict(reroute_depth=1, E=128, k=65), 2),
    (dict(n_groups=3), 1), (dict(n_groups=4, topk_groups=0), 1), (dict(n_groups=4, topk_groups=5), 1),
    (dict(n_groups=4, topk_groups=1, k=3), 1), (dict(n_groups=4, topk_groups=1, reroute_depth=1), 1),
    (dict(w_dtype=W.DT_INT4, d=384), 2), (dict(w_dtype=W.DT_INT4, F=192), 2),
    (dict(w_dtype=W.DT_INT4, act_dtype=W.DT_F32), 2),
])
def test_invalid_configs_rejected(L, kw, status):
    cfg = _cfg(L, **kw)
    n = ctypes.c_size_t(0)
    st = L.lib().moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n))
    assert st == status
    assert L.lib().moe_last_error()  # a description is set


def test_entry_points_validate_before_launch(L):
    lib = L.lib()
    cfg = _cfg(L)
    dummy = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation first
    big = ctypes.c_size_t(1 << 40)
    # missing required pointers
    assert lib.moe_route(ctypes.byref(cfg), None, None, None, None, None, None, None, dummy, big, None) == 1
    # a bias is required exactly when bias_mode != NONE
    assert lib.moe_route(ctypes.byref(cfg), dummy, dummy, dummy, None, None, dummy, dummy, dummy, big, None) == 1
    cfgb = _cfg(L, bias_mode=W.BIAS_LOGIT)
    assert lib.moe_route(ctypes.byref(cfgb), dummy, dummy, None, None, None, dummy, dummy, dummy, big, None) == 1
    # Gumbel noise with sigmoid scoring is unsupported
    cfgs = _cfg(L, score=W.SCORE_SIGMOID)
    assert lib.moe_route(ctypes.byref(cfgs), dummy, dummy, None, dummy, None, dummy, dummy, dummy, big, None) == 2
    # misaligned x
    assert lib.moe_route(ctypes.byref(cfg), ctypes.c_void_p(258), dummy, None, None, None, dummy, dummy, dummy, big,
                         None) == 1
    # the bf16 router needs its workspace
    assert lib.moe_route(ctypes.byref(cfg), dummy, dummy, None, None, None, dummy, dummy, dummy, 64, None) == 3
    assert lib.moe_route(ctypes.byref(cfg), dummy, dummy, None, None, None, dummy, dummy, None, 0, None) == 1
    # workspace too small / missing / misaligned
    args = [dummy] * 8
    assert lib.moe_permute(ctypes.byref(cfg), *args, dummy, 16, None) == 3
    assert lib.moe_permute(ctypes.byref(cfg), *args, None, 0, None) == 1
    assert lib.moe_permute(ctypes.byref(cfg), *args, ctypes.c_void_p(272), 1 << 40, None) == 1
    # expert weights: fp8 requires scales, bf16 forbids them; shared weights iff n_shared
    w = L.moe_expert_weights(256, 256, 256, None, None, None, None, None, None, None, None, None)
    cfg8 = _cfg(L, w_dtype=W.DT_FP8)
    assert lib.moe_expert_ffn(ctypes.byref(cfg8), dummy, dummy, dummy, ctypes.byref(w), dummy, None,
                              dummy, 1 << 40, None) == 1
    # INT4 requires its group words, 4-byte aligned
    cfg4 = _cfg(L, w_dtype=W.DT_INT4)
    assert lib.moe_expert_ffn(ctypes.byref(cfg4), dummy, dummy, dummy, ctypes.byref(w), dummy, None,
                              dummy, 1 << 40, None) == 1
    w4 = L.moe_expert_weights(256, 256, 256, 512, 512, 514, None, None, None, None, None, None)
    assert lib.moe_expert_ffn(ctypes.byref(cfg4), dummy, dummy, dummy, ctypes.byref(w4), dummy, None,
                              dummy, 1 << 40, None) == 1
    cfgsh = _cfg(L, n_shared=1)
    assert lib.moe_expert_ffn(ctypes.byref(cfgsh), dummy, dummy, dummy, ctypes.byref(w), dummy, dummy,
                              dummy, 1 << 40, None) == 1
    # forward: workspace too small
    assert lib.moe_forward(ctypes.byref(cfg), dummy, dummy, None, None, ctypes.byref(w), dummy, None,
                           None, dummy, 1024, None) == 3
    # balancing statistics: counts / prob_mean required, a logit bias needs the vector,
    # Gumbel noise needs softmax scoring, the partials need workspace
    assert lib.moe_router_stats(ctypes.byref(cfg), dummy, None, None, None, dummy, None, dummy, big, None) == 1
    assert lib.moe_router_stats(ctypes.byref(cfgb), dummy, None, None, dummy, dummy, None, dummy, big, None) == 1
    assert lib.moe_router_stats(ctypes.byref(cfgs), dummy, None, dummy, dummy, dummy, None, dummy, big, None) == 1
    assert lib.moe_router_stats(ctypes.byref(cfg), dummy, None, None, dummy, dummy, None, dummy, 8, None) == 3
    assert lib.moe_bias_update(ctypes.byref(cfg), dummy, None, ctypes.c_float(0.99), ctypes.c_float(0.01),
                               None) == 1
    assert lib.moe_bias_update(ctypes.byref(cfg), dummy, dummy, ctypes.c_float(float("nan")),
                               ctypes.c_float(0.01), None) == 1


def test_workspace_and_rows(L):
    s = W.WORKLOADS["skewed_fp8"]
    cfg = L.make_config(s)
    assert L.permuted_rows(cfg) == min(16384 * 2, 320 * 128)
    cfgd = L.make_config(W.WORKLOADS["skewed_fp8_decode"])
    assert L.permuted_rows(cfgd) == min(64, 1 * 128)
    big = L.workspace_bytes(L.make_config(W.WORKLOADS["fine_shared_bf16"]))
    assert big > 65536 * 7168 * (2 + 4)  # holds at least the bf16 x_perm and the f32 y_perm
    assert L.workspace_bytes(_cfg(L, T=0)) >= 0


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The binding has no fallback: a missing library is an ImportError."""
    import importlib.util
    import shutil
    pkg = os.path.join(ROOT, "mixture_experts_sparse_amd")
    dst = tmp_path / "mixture_experts_sparse_amd"
    dst.mkdir()
    for f in ["__init__.py", "_lib.py", "workloads.py"]:
        shutil.copy(os.path.join(pkg, f), dst / f)
    monkeypatch.syspath_prepend(str(tmp_path))
    for m in [m for m in list(__import__("sys").modules) if m.startswith("mixture_experts_sparse_amd")]:
        monkeypatch.delitem(__import__("sys").modules, m)
    mod = importlib.import_module("mixture_experts_sparse_amd")
    with pytest.raises(ImportError):
        mod.load()


@pytest.mark.parametrize("cf", [1e15, 1e30, 3.0e38])
def test_huge_capacity_factor_limits_nothing(L, cf):
    """A finite but enormous capacity factor makes C larger than any expert can
    be offered (T*k pairs): it must act as no limit, with every pair kept and
    the same row count and workspace as without a limit -- not an overflowed
    negative C * E."""
    s = W.WORKLOADS["fine_shared_bf16"]
    unlimited = L.make_config(s.replace(capacity_factor=0.0))
    huge = L.make_config(s.replace(capacity_factor=cf))
    assert L.permuted_rows(huge) == s.T * s.k == L.permuted_rows(unlimited)
    assert L.workspace_bytes(huge) == L.workspace_bytes(unlimited)
    tiny = L.make_config(s.replace(T=1, capacity_factor=cf))
    assert L.permuted_rows(tiny) == s.k


def test_noalloc_refuses_before_touching_the_device(L):
    """A layer whose workspace exceeds the allocation-free entry point's scratch
    is refused from the sizes alone (no device call: this runs without a GPU)."""
    lib = L.lib()
    cfg = _cfg(L)  # the Mixtral-shaped layer: hundreds of MiB of intermediates
    assert L.workspace_bytes(cfg) > L.MOE_NOALLOC_SCRATCH_BYTES
    d = ctypes.c_void_p(256)  # never dereferenced
    w = L.moe_expert_weights(256, 256, 256, None, None, None, None, None, None, None, None, None)
    st = lib.moe_forward_noalloc(ctypes.byref(cfg), d, d, None, None, ctypes.byref(w), d, None, None, None)
    assert st == 2  # MOE_ERR_UNSUPPORTED
    assert b"scratch" in lib.moe_last_error()
    # an invalid config is reported as such first
    bad = _cfg(L, k=0)
    assert lib.moe_forward_noalloc(ctypes.byref(bad), d, d, None, None, ctypes.byref(w), d, None, None, None) == 1
