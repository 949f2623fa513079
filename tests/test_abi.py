"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/moe.h declares, sizes workspaces, and rejects bad arguments
before touching the device (every call here fails validation, so nothing is
enqueued)."""
import ctypes
import json
import os
import re
import subprocess

import pytest

import sparse_mixture_experts_04_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward"):
        assert n in names
    assert set(names) == set(moe.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(moe.LIB, n)


def test_status_strings():
    for s in range(5):
        assert moe.status_string(s).startswith("MOE_")
    assert "unknown" in moe.status_string(99)
    assert "gfx950" in moe.version()


def _cfg(**kw):
    base = dict(T=64, d=128, F=256, E=8, k=2, capacity=-1, dtype="f32")
    base.update(kw)
    return moe.config(base["T"], base["d"], base["F"], base["E"], base["k"], base["capacity"], base["dtype"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(E=0, k=1), moe.MOE_ERR_INVALID_ARG),
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(E=65, k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(d=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(F=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(d=0), moe.MOE_ERR_INVALID_ARG),
])
def test_bad_config_rejected(kw, status):
    cfg = _cfg(**kw)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD)
    assert ei.value.status == status
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(cfg, 1, 1, None, 1, 1, stream=0)
    assert ei.value.status == status


def test_bad_dtype_and_op():
    cfg = _cfg()
    cfg.dtype = 7
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD)
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_size(_cfg(), 17)


def test_null_pointers_rejected():
    cfg = _cfg()
    calls = [
        lambda: moe.moe_route(cfg, None, 1, None, 1, 1, stream=0),
        lambda: moe.moe_route(cfg, 1, 1, None, None, 1, stream=0),
        lambda: moe.moe_dispatch(cfg, None, 1, 1, 1, 1, 1, 1, 1, 1 << 30, stream=0),
        lambda: moe.moe_dispatch(cfg, 1, 1, None, 1, 1, 1, 1, 1, 1 << 30, stream=0),
        lambda: moe.moe_expert_up(cfg, 1, None, 1, 1, stream=0),
        lambda: moe.moe_expert_down(cfg, 1, 1, None, 1, stream=0),
        lambda: moe.moe_expert_ffn(cfg, 1, 1, 1, 1, None, 1, 1 << 30, stream=0),
        lambda: moe.moe_combine(cfg, 1, None, 1, 1, stream=0),
        lambda: moe.moe_forward(cfg, 1, 1, None, 1, 1, None, 1, 1, 1, 1, 1, 1, 1, 1 << 30, stream=0),
    ]
    for c in calls:
        with pytest.raises(moe.MoeError) as ei:
            c()
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_workspace_too_small_rejected():
    cfg = _cfg(capacity=5)
    need = moe.moe_workspace_size(cfg, moe.MOE_OP_DISPATCH)
    assert need > 0
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_dispatch(cfg, 1, 1, 1, 1, 1, 1, 1, 1, need - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    need_f = moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward(cfg, 1, 1, None, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, need_f - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    need_h = moe.moe_workspace_size(cfg, moe.MOE_OP_EXPERT_FFN)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_expert_ffn(cfg, 1, 1, 1, 1, 1, 1, need_h - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL


def test_route_workspace():
    # small T with a large hidden size splits the gate projection over K
    cfg = moe.config(8, 3584, 2560, 64, 2, -1, "bf16")
    need = moe.moe_workspace_size(cfg, moe.MOE_OP_ROUTE)
    gate_t = 64 * 3584 * 2
    assert need > gate_t and (need - gate_t) % (8 * 64 * 4) == 0
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route(cfg, 1, 1, None, 1, 1, 1, need - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    # plenty of tokens: one pass, only the transposed gate
    assert moe.moe_workspace_size(moe.config(8192, 2048, 5632, 32, 2), moe.MOE_OP_ROUTE) == 32 * 2048 * 2


def test_workspace_sizes():
    T, d, F, E, k = 8192, 2048, 5632, 32, 2
    cfg = moe.config(T, d, F, E, k, -1, "bf16")
    h = moe.moe_workspace_size(cfg, moe.MOE_OP_EXPERT_FFN)
    assert h == T * k * F * 2
    fwd = moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD)
    disp = moe.moe_workspace_size(cfg, moe.MOE_OP_DISPATCH)
    assert fwd >= disp + 2 * T * k * d * 2 + h
    capcfg = moe.config(T, d, F, E, k, 1024, "bf16")
    assert moe.moe_workspace_size(capcfg, moe.MOE_OP_DISPATCH) > disp
    # T = 0 is valid and needs (almost) nothing
    assert moe.moe_workspace_size(moe.config(0, d, F, E, k), moe.MOE_OP_EXPERT_FFN) == 0


def test_gathered_up_projection_support():
    # bf16 with experts that may hold more than 64 pairs (min(T, C) > 64): the 256x256 kernel
    assert moe.moe_expert_up_gather_supported(moe.config(8192, 2048, 5632, 32, 2, -1, "bf16"))
    assert moe.moe_expert_up_gather_supported(moe.config(65, 128, 128, 8, 2, -1, "bf16"))
    assert moe.moe_expert_up_gather_supported(moe.config(32768, 2048, 1408, 32, 4, 4096, "bf16"))
    assert not moe.moe_expert_up_gather_supported(moe.config(8192, 2048, 5632, 32, 2, 64, "bf16"))
    assert not moe.moe_expert_up_gather_supported(moe.config(8192, 2048, 5632, 32, 2, -1, "f32"))
    # decode-sized batches gather too, where the decode kernel runs: at most 16 pairs per expert, or at
    # most 64 with at most 16 pairs per expert on average (T * k <= 16 E)
    assert moe.moe_expert_up_gather_supported(moe.config(8, 3584, 2560, 64, 2, -1, "bf16"))
    assert moe.moe_expert_up_gather_supported(moe.config(300, 1024, 256, 16, 2, 16, "bf16"))
    assert moe.moe_expert_up_gather_supported(moe.config(64, 128, 128, 8, 2, -1, "bf16"))  # 128 pairs = 16 E
    assert moe.moe_expert_up_gather_supported(moe.config(64, 3584, 2560, 64, 2, -1, "bf16"))
    assert not moe.moe_expert_up_gather_supported(moe.config(64, 128, 128, 4, 2, -1, "bf16"))  # 128 pairs > 16 E
    assert not moe.moe_expert_up_gather_supported(moe.config(300, 1024, 256, 16, 2, 17, "bf16"))  # 600 > 16 E
    assert not moe.moe_expert_up_gather_supported(moe.config(8, 3520, 2560, 64, 2, -1, "bf16"))  # d % 128 != 0
    assert not moe.moe_expert_up_gather_supported(moe.config(8, 3584, 2560, 64, 2, -1, "f32"))
    # X must fit 32-bit buffer offsets: T * d * 2 < 2^31
    assert moe.moe_expert_up_gather_supported(moe.config((1 << 31) // 8192 - 1, 4096, 128, 8, 2, -1, "bf16"))
    assert not moe.moe_expert_up_gather_supported(moe.config((1 << 31) // 8192, 4096, 128, 8, 2, -1, "bf16"))
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_expert_up_gather_supported(_cfg(k=9))
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_gathered_up_projection_rejects_before_launch():
    cfg = moe.config(300, 128, 128, 8, 2, -1, "bf16")
    for args in [(None, 1, 1, 1, 1), (1, None, 1, 1, 1), (1, 1, None, 1, 1), (1, 1, 1, None, 1), (1, 1, 1, 1, None)]:
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_expert_up_gather(cfg, *args, stream=0)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    for unsupported in (moe.config(64, 128, 128, 4, 2, -1, "bf16"), moe.config(300, 128, 128, 8, 2, -1, "f32")):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_expert_up_gather(unsupported, 1, 1, 1, 1, 1, stream=0)
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    # T = 0 is a no-op for any pointers
    moe.moe_expert_up_gather(moe.config(0, 128, 128, 8, 2, -1, "bf16"), None, None, None, None, None, stream=0)


def test_route_stats_rejects_before_launch():
    cfg = moe.config(64, 128, 256, 8, 2, -1, "bf16")
    need = moe.moe_workspace_size(cfg, moe.MOE_OP_ROUTE_STATS)
    assert need >= moe.moe_workspace_size(cfg, moe.MOE_OP_ROUTE) + 4 * 8 * 4  # 4 tiles of 16 tokens x E floats
    for tau in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_route_stats(cfg, 1, 1, None, tau, 1, 1, 1, 1, 1, 1, need, stream=0)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    for i in range(7):
        args = [1] * 7
        args[i] = None
        X, Wg, ids, w, pm, sf, aux = args
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_route_stats(cfg, X, Wg, None, 1.0, ids, w, pm, sf, aux, 1, need, stream=0)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route_stats(cfg, 1, 1, None, 1.0, 1, 1, 1, 1, 1, 1, need - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    # T = 0: nothing to do, any pointers
    moe.moe_route_stats(moe.config(0, 128, 256, 8, 2), None, None, None, 1.0, None, None, None, None, None, stream=0)


def test_capacity_from_factor_matches_oracle():
    import oracle
    for c in json.load(open(os.path.join(ROOT, "tests", "golden", "capacity_factor_example.json"),
                            encoding="utf-8"))["cases"]:
        assert moe.moe_capacity_from_factor(c["batch"], c["seq_len"], c["E"], c["k"], c["factor"]) == c["C"]
    for batch in (0, 1, 3, 16, 300):
        for seq in (0, 1, 2, 7, 512, 4096):
            for E, k in ((1, 1), (8, 2), (32, 4), (64, 8)):
                for f in (0.5, 1.0, 1.25, 2.0, 4.0):
                    assert moe.moe_capacity_from_factor(batch, seq, E, k, f) == \
                        oracle.expert_capacity_from_factor(batch, seq, E, k, f), (batch, seq, E, k, f)
    for bad in ((-1, 8, 8, 2, 2.0), (1, -1, 8, 2, 2.0), (1, 8, 0, 1, 2.0), (1, 8, 8, 9, 2.0), (1, 8, 8, 2, 0.0),
                (1, 8, 8, 2, float("inf"))):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_capacity_from_factor(*bad)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_reroute_entry_points_reject_before_launch():
    cfg = moe.config(300, 128, 256, 8, 2, 40, "bf16")
    need_d = moe.moe_workspace_size(cfg, moe.MOE_OP_DISPATCH_REROUTE)
    # the rerouted assignment (T*k int32) on top of the capacity dispatch's scratch
    assert need_d >= moe.moe_workspace_size(cfg, moe.MOE_OP_DISPATCH) + 300 * 2 * 4
    need_f = moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD_REROUTE)
    assert need_f >= moe.moe_workspace_size(cfg, moe.MOE_OP_FORWARD) + 300 * 2 * 4
    calls = [
        lambda: moe.moe_route_ranked(cfg, 1, 1, None, 1, 1, None, 1, 1 << 30, stream=0),
        lambda: moe.moe_route_ranked(cfg, None, 1, None, 1, 1, 1, 1, 1 << 30, stream=0),
        lambda: moe.moe_dispatch_reroute(cfg, 1, None, 1, 1, 1, 1, 1, 1, 1, need_d, stream=0),
        lambda: moe.moe_dispatch_reroute(cfg, None, 1, 1, 1, 1, 1, 1, 1, 1, need_d, stream=0),
        lambda: moe.moe_dispatch_reroute(cfg, 1, 1, 1, None, 1, 1, 1, 1, 1, need_d, stream=0),
        lambda: moe.moe_forward_reroute(cfg, 1, 1, None, 1, 1, 1, 1, 1, None, 1, 1, 1, 1, 1, need_f, stream=0),
        lambda: moe.moe_forward_reroute(cfg, 1, 1, None, 1, 1, None, 1, 1, 1, 1, 1, 1, 1, 1, need_f, stream=0),
    ]
    for c in calls:
        with pytest.raises(moe.MoeError) as ei:
            c()
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_dispatch_reroute(cfg, 1, 1, 1, 1, 1, 1, 1, 1, 1, need_d - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_reroute(cfg, 1, 1, None, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, need_f - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    # T = 0: nothing to do
    moe.moe_route_ranked(moe.config(0, 128, 256, 8, 2), None, None, None, None, None, None, stream=0)


def test_binding_rejects_bad_tensors_before_the_library():
    """The library cannot see buffer sizes, so the binding checks every
    tensor against moe.h's documented device, dtype, contiguity and size
    before passing its pointer (no call reaches the library here)."""
    import torch
    cfg = moe.config(16, 128, 256, 8, 2, -1, "bf16")
    ok = dict(X=torch.empty(16, 128, dtype=torch.bfloat16), Wg=torch.empty(128, 8, dtype=torch.bfloat16))
    # a CPU tensor is refused (it is not device memory)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_route(cfg, ok["X"], ok["Wg"], None, 1, 1, 1, 1 << 20, stream=0)
    meta = lambda shape, dt: torch.empty(shape, dtype=dt, device="meta")  # noqa: E731
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_combine(cfg, meta((32, 128), torch.bfloat16), 1, 1, 1, stream=0)
    # int pointers pass through unchecked: the library then validates nulls
    with pytest.raises(moe.MoeError):
        moe.moe_combine(cfg, 1, None, 1, 1, stream=0)


def test_binding_arg_checks():
    """The per-buffer check itself: dtype, contiguity and size are enforced
    for tensors; None, int pointers and empty requirements pass."""
    import torch
    from sparse_mixture_experts_04_amd import _lib

    class FakeCuda:  # stands in for a device tensor (no GPU here)
        def __init__(self, t):
            self.t = t
            self.device = torch.device("cuda", 0)
            self.dtype = t.dtype

        def is_contiguous(self):
            return self.t.is_contiguous()

        def numel(self):
            return self.t.numel()

    orig = _lib.torch.Tensor
    try:
        _lib.torch.Tensor = FakeCuda  # isinstance checks accept the stand-in
        good = FakeCuda(torch.empty(4, 8, dtype=torch.int32))
        _lib._arg("f", "a", good, torch.int32, 32)
        _lib._arg("f", "a", None, torch.int32, 32)
        _lib._arg("f", "a", 1234, torch.int32, 32)
        _lib._arg("f", "a", good, torch.float32, 0)
        with pytest.raises(TypeError, match="dtype"):
            _lib._arg("f", "a", good, torch.float32, 32)
        with pytest.raises(ValueError, match="needs 33"):
            _lib._arg("f", "a", good, torch.int32, 33)
        with pytest.raises(ValueError, match="contiguous"):
            _lib._arg("f", "a", FakeCuda(torch.empty(8, 4, dtype=torch.int32).t()), torch.int32, 32)
        with pytest.raises(TypeError):
            _lib._arg("f", "a", "not a tensor", torch.int32, 32)
    finally:
        _lib.torch.Tensor = orig
