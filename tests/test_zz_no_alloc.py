"""The workspace-free layer entry point (moe_layer_forward_static) against
moe_layer_forward, through the C ABI (needs an MI355X).

Two calls in a row on the library's per-GPU scratch, the second with fewer
tokens than the first, each checked against moe_layer_forward on the same
inputs: the same kernels run on the same values, so ids, weights and outputs
must agree bit for bit (which implies the oracle bar both already meet).
"""
import functools
import sys

import numpy as np
import pytest

from synth import WORKLOADS, make_layer, make_tokens
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")


def say(*a):
    print("[no-alloc]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def packed_of(wi: int):
    from quantized_expert_ffn_moe_amd import binding as B
    return B.pack_layer(make_layer(WORKLOADS[wi], 0))


def tokens(wi, n, batch):
    x, bits = make_tokens(WORKLOADS[wi], batch=batch, n_tokens=n)
    if bits is not None:
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def both(xt, packed, flags, y0=None):
    """(ids, w, y) of the static entry point and of moe_layer_forward."""
    from quantized_expert_ffn_moe_amd import binding as B
    T = xt.shape[0]
    outs = []
    for static in (True, False):
        y = torch.zeros(T, 1280, dtype=torch.float32, device="cuda") if y0 is None else y0.clone()
        ids = torch.full((T, 6), -1, dtype=torch.int32, device="cuda")
        w = torch.zeros(T, 6, dtype=torch.float32, device="cuda")
        if static:
            B.moe_layer_forward_static(xt, packed, y, ids, w, flags)
        else:
            B.moe_layer_forward(xt, packed, y, ids, w, B.workspace(T), flags)
        torch.cuda.synchronize()
        outs.append((ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()))
    return outs


def assert_same(a, b):
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("wi,counts", [(2, (200, 37)), (3, (256, 3)), (5, (130, 64))])
def test_static_entry_matches_workspace_entry_two_calls(lib, wi, counts):
    """Two calls in a row, the second smaller: bf16 int4 G32 with a biased
    router (grouped path, then a smaller grouped call), bf16 int4 G128 (the
    maximum, then the per-token path), f32 int4 G64 / int8 G128 with the norm
    and an in-place residual."""
    from quantized_expert_ffn_moe_amd import binding as B
    wl = WORKLOADS[wi]
    flags = 0
    for k, T in enumerate(counts):
        xt = tokens(wi, T, batch=40 + k)
        y0 = None
        if wl.x_dtype == "f32":
            flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE
            y0 = torch.from_numpy(np.random.default_rng(T).normal(0, 1, (T, 1280)).astype(np.float32)).cuda()
        a, b = both(xt, packed_of(wi), flags, y0)
        assert a[0].min() >= 0 and a[0].max() < 64
        assert_same(a, b)
        say(f"{wl.name}: call {k + 1} with {T} tokens identical to moe_layer_forward")


def test_static_entry_limits(lib):
    from quantized_expert_ffn_moe_amd import binding as B
    p = packed_of(2)
    for T, flags in ((257, 0), (19, B.MOE_FORCE_DECODE)):
        xt = tokens(2, T, batch=50)
        y = torch.empty(T, 1280, dtype=torch.float32, device="cuda")
        ids = torch.empty(T, 6, dtype=torch.int32, device="cuda")
        w = torch.empty(T, 6, dtype=torch.float32, device="cuda")
        with pytest.raises(B.MoeError, match="SHAPE"):
            B.moe_layer_forward_static(xt, p, y, ids, w, flags)
    # an empty call enqueues nothing
    y = torch.empty(0, 1280, dtype=torch.float32, device="cuda")
    B.moe_layer_forward_static(tokens(2, 0, batch=51), p, y, y.view(torch.int32)[:, :6], y[:, :6])
    # the per-token path still runs through it up to 18 tokens
    xt = tokens(2, 18, batch=52)
    a, b = both(xt, p, B.MOE_FORCE_DECODE)
    assert_same(a, b)
