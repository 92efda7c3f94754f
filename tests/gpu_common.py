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


class FfnMemo:
    """Memoised oracle expert outputs of one stack, keyed by (layer, expert,
    x bits): a teacher-forced and a free-running oracle pass over the same
    layer usually see the same bf16 x, and the float64 FFN at the 235B shape
    takes about half a second per expert."""

    def __init__(self, seed, dims):
        self.seed, self.dims = seed, dims
        self.experts = {}
        self.out = {}

    def layer(self, L):
        if L not in self.experts:
            self.experts[L] = LazyExperts(self.seed, self.dims, L)
        ex = self.experts[L]

        def ffn(e, x, xbits):
            key = (L, int(e), np.asarray(xbits).tobytes())
            if key not in self.out:
                self.out[key] = oracle.expert_ffn(ex[int(e)], x, self.dims.chunk)
            return self.out[key]
        return ex, ffn


def check_chain_against_oracle(dims, stack, h0, chain_out, per_layer_inputs, i_rec, w_rec, tag,
                               seed=1337, tie_tol=1e-4):
    """The oracle checks of a chained decode run.

    Teacher-forced (the parity protocol): each layer is recomputed from the
    GPU's own input residual; x bits and expert ids must match exactly, the
    weights to 2e-6 relative, and the layer's MoE delta must meet the output
    tolerance.  Free-running: the float64 oracle chain from h0; routing must
    agree layer by layer unless the first difference is a near-tie of the
    oracle's logits (then the chains legitimately diverge and the comparison
    stops); otherwise the final residual must be within the tolerance of the
    summed MoE deltas."""
    memo = FfnMemo(seed, dims)
    n_layers = len(per_layer_inputs)
    worst = 0.0
    for L in range(n_layers):
        ex, ffn = memo.layer(L)
        res_in = per_layer_inputs[L][0]
        ref = oracle.moe_layer(res_in.astype(np.float64), stack.router_bits[L], ex, dims, ffn=ffn)
        xb, ig, wg, r_out = per_layer_inputs[L][1]
        assert np.array_equal(xb, ref["x_bits"]), f"{tag} layer {L}: x bits"
        assert list(ig) == ref["idx"], f"{tag} layer {L}: ids {list(ig)} vs {ref['idx']}"
        assert np.allclose(wg, ref["w"], rtol=2e-6, atol=1e-7), f"{tag} layer {L}: weights"
        y = r_out.astype(np.float64) - res_in.astype(np.float64)
        worst = max(worst, check_moe_output(y, ref["y"], f"{tag} layer {L}"))
    say(f"[{tag}] teacher-forced worst rel-L2 {worst:.2e} over {n_layers} layers")
    ro = h0.astype(np.float64)
    for L in range(n_layers):
        ex, ffn = memo.layer(L)
        ref = oracle.moe_layer(ro, stack.router_bits[L], ex, dims, ffn=ffn)
        gi = [int(v) for v in i_rec[L]]
        if gi != ref["idx"]:
            assert topk_gap_ok(ref["logits"], gi, ref["idx"], dims.top_k, tie_tol), f"{tag} layer {L}"
            say(f"[{tag}] near-tie flip at layer {L}; free-running comparison stops")
            return worst
        ro = ref["r_out"]
    rel = np.linalg.norm(chain_out - ro) / np.linalg.norm(ro - h0)
    say(f"[{tag}] free-running final residual rel error (vs summed MoE deltas) {rel:.2e}")
    assert rel <= REL_L2, f"{tag}: free-running chain rel error {rel:.3e}"
    return worst


def oracle_chunk_outputs(res, router_bits, experts, dims, bias=None):
    """Oracle routing and MoE output of every token of a chunk, with each
    union expert's FFN evaluated once on all of its tokens' inputs (the
    oracle's expert_ffn applied to a matrix of column inputs, i.e. the same
    definition for every column).  Returns per-token dicts with x_bits, idx,
    w and y."""
    T = res.shape[0]
    toks = []
    by_expert = {}
    for t in range(T):
        x, xbits = oracle.rmsnorm_bf16(res[t].astype(np.float64), dims.rms_eps)
        l = oracle.router_logits(router_bits, x, bias)
        idx, w = oracle.select_topk(l, dims.top_k, dims.norm_topk_prob)
        toks.append({"x": x, "x_bits": xbits, "idx": idx, "w": w})
        for e in idx:
            by_expert.setdefault(int(e), []).append(t)
    outs = {}
    for e, ts in by_expert.items():
        X = np.stack([toks[t]["x"] for t in ts], axis=1)          # [d][n]
        Y = oracle.expert_ffn(experts[e], X, dims.chunk)           # [d][n]
        for c, t in enumerate(ts):
            outs[(e, t)] = Y[:, c]
    for t, tk in enumerate(toks):
        y = np.zeros(dims.d_model, dtype=np.float64)
        for r, e in enumerate(tk["idx"]):                          # rank order
            y = y + tk["w"][r] * outs[(int(e), t)]
        tk["y"] = y
    return toks


def check_prefill_against_oracle(got, res, stack, dims, layer, tag):
    """Every token of a prefill chunk against the oracle: ids exact, weights to
    2e-6 relative, MoE output within the tolerance."""
    bias = None if stack.bias_np is None else stack.bias_np[layer]
    toks = oracle_chunk_outputs(res, stack.router_bits[layer], LazyExperts(stack.seed, dims, layer), dims, bias)
    worst = 0.0
    for t, ref in enumerate(toks):
        assert got["idx"][t].tolist() == ref["idx"], f"{tag} token {t}"
        assert np.allclose(got["w"][t], ref["w"], rtol=2e-6, atol=1e-7), f"{tag} token {t}: weights"
        y = got["r_out"][t].astype(np.float64) - res[t].astype(np.float64)
        worst = max(worst, check_moe_output(y, ref["y"], f"{tag} t{t}"))
    say(f"[{tag}] {len(toks)} tokens, worst rel-L2 {worst:.2e}")
    return worst
