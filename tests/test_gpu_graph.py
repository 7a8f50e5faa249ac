"""A whole layer step (route, permute, expert forward, combine) captured in a
HIP graph through torch.cuda.CUDAGraph: the library launches on the caller's
stream and allocates, synchronises and clears nothing itself, so the step can
be captured as it is. Every replay must equal the eager result bit for bit,
with other eager work and synchronisations between the replays and the
outputs overwritten before each one."""
import numpy as np
import pytest
import torch

from bit_mixture_experts_amd import inputs as inp
from gpu_helpers import DEV, run_layer, to_dev

pytestmark = pytest.mark.gpu
moe4 = pytest.importorskip("bit_mixture_experts_amd.moe4")

from test_gpu_parity import GPTOSS_SMALL, QWEN_SMALL, layer_of  # noqa: E402

CASES = [(QWEN_SMALL, 5), (QWEN_SMALL, 100), (GPTOSS_SMALL, 3), (GPTOSS_SMALL, 200)]


class CapturedStep:
    """Buffers of one step and the step itself, for eager calls and capture."""

    def __init__(self, ex, spec, T):
        E, H, k = spec.E, spec.H, spec.k
        S = T * k
        self.ex, self.k, self.E = ex, k, E
        self.x = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        self.lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
        self.w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        self.sor = torch.empty(S, dtype=torch.int32, device=DEV)
        self.ros = torch.empty(S, dtype=torch.int32, device=DEV)
        self.x_perm = torch.empty((S, H), dtype=torch.bfloat16, device=DEV)
        self.y_perm = torch.empty((S, H), dtype=torch.float32, device=DEV)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        self.ws = torch.empty(moe4.moe4_workspace_size(ex, T, k), dtype=torch.uint8,
                              device=DEV)

    def __call__(self):
        moe4.moe4_route(self.lg, self.k, self.idx, self.w)
        moe4.moe4_permute(self.idx, self.E, self.offsets, self.sor, self.ros, x=self.x,
                          x_perm=self.x_perm, ws=self.ws)
        moe4.moe4_expert_forward(self.ex, self.x_perm, self.offsets, self.y_perm, ws=self.ws)
        moe4.moe4_combine(self.y_perm, self.ros, self.w, self.out, self.k)

    def scramble(self):
        """Overwrite every output with garbage (eagerly, outside the graph)."""
        for t in (self.idx, self.offsets, self.sor, self.ros):
            t.fill_(-7)
        self.w.fill_(float("nan"))
        self.x_perm.fill_(float("nan"))
        self.y_perm.fill_(float("nan"))
        self.out.fill_(float("nan"))


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("spec,T", CASES, ids=[f"{s.name}-T{t}" for s, t in CASES])
def test_forward_graph_replays(spec, T):
    L = layer_of(spec)
    ex = L.device()
    x, lg = inp.host_tokens(spec, T)
    x2, lg2 = inp.host_tokens(spec, T, seed=11)
    eager = run_layer(ex, to_dev(x), to_dev(lg), spec.k)
    st = CapturedStep(ex, spec, T)
    st.x.copy_(to_dev(x))
    st.lg.copy_(to_dev(lg))
    st()   # outside capture first: the library's one-time kernel attributes
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st()
    torch.cuda.synchronize()
    for r in range(4):
        st.scramble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(st.idx, eager["idx"]), f"replay {r}: idx"
        assert _same(st.offsets, eager["offsets"]), f"replay {r}: offsets"
        assert _same(st.ros, eager["row_of_slot"]), f"replay {r}: row_of_slot"
        assert _same(st.y_perm, eager["y_perm"]), f"replay {r}: y_perm"
        assert _same(st.out, eager["out"]), f"replay {r}: out"
        # eager work on other tokens between replays
        other = run_layer(ex, to_dev(x2), to_dev(lg2), spec.k)
        assert np.isfinite(other["out32"].cpu().numpy()).all()
