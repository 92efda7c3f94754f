"""Helpers shared by the GPU parity tests (not collected as tests)."""
import numpy as np
import pytest
import torch

import oracle
import synth

REL_L2 = 2e-3       # rel-L2 bound on the MoE output per token and layer
MAX_ABS = 1e-2      # max-abs bound, relative to max |reference|


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, flush=True)


class LazyExperts(dict):
    """expert index -> logical expert of one layer, drawn on first use."""

    def __init__(self, seed, dims, layer):
        super().__init__()
        self.seed, self.dims, self.layer = seed, dims, layer

    def __missing__(self, e):
        v = synth.expert_logical(self.seed, self.dims, self.layer, int(e))
        self[e] = v
        return v


def check_moe_output(y_gpu, y_ref, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rel = np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    mx = np.max(np.abs(y_gpu - y_ref))
    bound = MAX_ABS * np.max(np.abs(y_ref))
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mx <= bound, f"{what}: max-abs {mx:.3e} > {bound:.3e}"
    return rel


def bits_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def random_residual(rng, n_tok, d, scale=1.0):
    return (rng.standard_normal((n_tok, d)) * scale).astype(np.float32)


def topk_gap_ok(logits, idx_gpu, idx_ref, k, tol):
    """A routing difference is acceptable only if it is a near-tie: the
    oracle's logits at the first differing rank are within tol."""
    l = np.asarray(logits)
    for r in range(k):
        if idx_gpu[r] != idx_ref[r]:
            return abs(l[idx_gpu[r]] - l[idx_ref[r]]) <= tol
    return True
