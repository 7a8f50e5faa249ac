"""The no-allocation expert forward against the workspace forward, through the
C ABI: the same outputs bit for bit (both run the same kernels; the scratch
only replaces the caller's workspace), on two calls in a row, the second with
a smaller input, on every kernel path that uses scratch (bf16 h for both
families, the adapter projection, a double-quantised stack); and the calls
that need more scratch than the library holds are refused before anything
runs."""
import numpy as np
import pytest
import torch

import oracle
from bit_mixture_experts_amd import inputs as inp
from tests.gpu_helpers import DEV, HostLayer, assert_close, run_layer, say, to_dev

pytestmark = pytest.mark.gpu

moe4 = pytest.importorskip("bit_mixture_experts_amd.moe4")

LORA = inp.QWEN3_30B_NF4_LORA.scaled(name="noalloc_lora_nf4", seed_id=140, E=8, k=2, H=256,
                                     I=128, tokens=(150, 20))
MXFP4 = inp.GPT_OSS_20B_MXFP4.scaled(name="noalloc_mxfp4", seed_id=141, E=8, k=4, H=352, I=352,
                                     tokens=(200, 3))


def _routed(spec, T, L):
    x, lg = inp.host_tokens(spec, T)
    res = run_layer(L.device(), to_dev(x), to_dev(lg), spec.k)
    return x, lg, res


def _both(ex, res, lora_r):
    """Workspace forward and no-allocation forward on the same rows."""
    S, H = res["x_perm"].shape
    outs = []
    for noalloc in (False, True):
        y = torch.full((S, H), float("nan"), dtype=torch.float32, device=DEV)
        gu = torch.full((S, 2 * ex.I), float("nan"), dtype=torch.float32, device=DEV)
        xa = (torch.full((S, lora_r), float("nan"), dtype=torch.float32, device=DEV)
              if lora_r else None)
        if noalloc:
            moe4.moe4_expert_forward_noalloc(ex, res["x_perm"], res["offsets"], y, save_gu=gu,
                                             save_xa=xa)
        else:
            ws = torch.empty(moe4.moe4_workspace_size(ex, S, 1), dtype=torch.uint8, device=DEV)
            moe4.moe4_expert_forward(ex, res["x_perm"], res["offsets"], y, save_gu=gu,
                                     save_xa=xa, ws=ws)
        torch.cuda.synchronize()
        outs.append((y, gu, xa, moe4.moe4_last_variant()))
    return outs


def _check_equal(a, b, what):
    for name, ta, tb in (("y_perm", a[0], b[0]), ("save_gu", a[1], b[1]), ("save_xa", a[2], b[2])):
        if ta is None:
            continue
        assert torch.equal(ta, tb), f"{what}: {name} differs from the workspace forward"
    assert a[3] == b[3], f"{what}: kernel family {a[3]} vs {b[3]}"


@pytest.mark.parametrize("spec", [LORA, MXFP4], ids=["nf4_lora", "mxfp4"])
def test_noalloc_forward_matches_workspace_forward(spec):
    L = HostLayer(spec)
    for variant in (moe4.MOE4_VARIANT_TILED, moe4.MOE4_VARIANT_SKINNY):
        for T in spec.tokens:   # two calls in a row, the second smaller
            say(f"no-allocation forward: {spec.name} T={T} variant={variant}")
            x, lg, res = _routed(spec, T, L)
            ex = L.device(variant)
            ws_out, na_out = _both(ex, res, spec.lora_r)
            _check_equal(ws_out, na_out, f"{spec.name} T={T} v{variant}")
            # and the result is the layer's: against the oracle
            ri, rw = oracle.route(lg, spec.k)
            ref = oracle.layer_forward(x, ri, rw, L.W, keep=True)
            assert_close(na_out[0].cpu().numpy(), ref["y"], "y_perm (no allocation)")


def test_noalloc_forward_double_quant_tiled():
    """A double-quantised stack on the prefill-sized kernel (both absmax levels
    decoded per k-tile) gives the workspace entry point's results bit for bit."""
    from tests.test_gpu_parity import DQLayer, QWEN_SMALL
    D = DQLayer(QWEN_SMALL)
    for T in (100, 5):
        say(f"no-allocation forward, double-quantised: T={T}")
        x, lg = inp.host_tokens(QWEN_SMALL, T)
        ex = D.device(moe4.MOE4_VARIANT_TILED)
        res = run_layer(ex, to_dev(x), to_dev(lg), QWEN_SMALL.k)
        ws_out, na_out = _both(ex, res, 0)
        _check_equal(ws_out, na_out, f"double-quantised T={T}")


def test_noalloc_forward_refuses_oversized_calls():
    L = HostLayer(inp.TINY_NF4)
    ex = L.device()
    # h alone needs rows * I * 2 bytes: past the scratch for rows > 16 MiB / (2 I)
    rows = moe4.MOE4_NOALLOC_SCRATCH_BYTES // (2 * ex.I) + 1
    xp = torch.empty((rows, ex.H), dtype=torch.bfloat16, device=DEV)
    yp = torch.empty((rows, ex.H), dtype=torch.float32, device=DEV)
    offsets = torch.zeros(ex.E + 1, dtype=torch.int32, device=DEV)
    with pytest.raises(moe4.Moe4Error) as err:
        moe4.moe4_expert_forward_noalloc(ex, xp, offsets, yp)
    assert err.value.code == moe4.MOE4_EWORKSPACE and "scratch" in str(err.value)
