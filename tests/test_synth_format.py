"""The seeded input generator and the SMOE-Q4 blob encoding (CPU)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("wl, blob, stride", [
    (synth.CONFIGS[0], 61440, 65536),
    (synth.CONFIGS[1], 2654208, 162 * 16384),
    (synth.CONFIGS[2], 10616832, 648 * 16384),
])
def test_blob_sizes_exact(wl, blob, stride):
    off = synth.blob_sections(wl.dims)
    assert off["bytes"] == blob and off["stride"] == stride
    assert off["stride"] % synth.BLOB_ALIGN == 0
    for k, v in off.items():
        assert v % 16 == 0, k


def test_vault_bytes_per_token():
    # Q4 expert bytes one decode token touches: layers * top_k * blob bytes.
    w1, w2 = synth.CONFIGS[1], synth.CONFIGS[2]
    assert w1.n_layers * w1.dims.top_k * synth.blob_sections(w1.dims)["bytes"] == 1019215872
    assert w2.n_layers * w2.dims.top_k * synth.blob_sections(w2.dims)["bytes"] == 7983857664
    assert w2.n_layers * w2.dims.n_experts * synth.blob_sections(w2.dims)["stride"] == 127741722624


def test_nibble_and_param_layout():
    dims = synth.Dims(256, 128, 16, 4, 32)
    off = synth.blob_sections(dims)
    blob = synth.pack_blob(1337, dims, 0, 3)
    for name, mat, rows, cols in (("gate", 0, 128, 256), ("up", 1, 128, 256), ("down", 2, 256, 128)):
        q = synth.expert_codes(1337, dims, 0, 3, mat)
        sb, mb = synth.expert_params_bits(1337, dims, 0, 3, mat)
        for n, j in ((0, 0), (5, 17), (rows - 1, cols // 2 - 1)):
            byte = blob[off[name + "_codes"] + n * cols // 2 + j]
            assert byte & 15 == q[n, 2 * j] and byte >> 4 == q[n, 2 * j + 1]
        nc = cols // dims.chunk
        for n, c in ((0, 0), (7, nc - 1), (rows - 1, 1)):
            p = off[name + "_params"] + (n * nc + c) * 4
            assert int(blob[p]) | int(blob[p + 1]) << 8 == sb[n, c]
            assert int(blob[p + 2]) | int(blob[p + 3]) << 8 == mb[n, c]
    assert np.all(blob[off["bytes"]:] == 0)


def test_two_packers_agree():
    dims = synth.Dims(512, 96, 8, 2, 64)
    a = synth.pack_blob(7, dims, 2, 5)
    b = synth.pack_logical(dims, synth.expert_logical(7, dims, 2, 5))
    assert np.array_equal(a, b)


def test_distributions():
    dims = synth.Dims(2048, 768, 128, 8, 64)
    q = synth.expert_codes(1337, dims, 1, 2, synth.MAT_GATE)
    freq = np.bincount(q.reshape(-1), minlength=16) / q.size
    assert np.all(np.abs(freq - 1 / 16) < 0.002)
    sb, mb = synth.expert_params_bits(1337, dims, 1, 2, synth.MAT_DOWN)
    s, m = oracle.bf16_to_f64(sb), oracle.bf16_to_f64(mb)
    assert s.min() >= 0.002 - 1e-5 and s.max() <= 0.01 + 1e-4
    assert np.array_equal(m, -8 * s)
    w = oracle.bf16_to_f64(synth.router_bits(1337, dims, 0))
    assert abs(w.std() - 0.02) < 0.0005 and abs(w.mean()) < 0.0005
    h = synth.hidden_bf16(1337, 0, 4096)
    assert abs(h.std() - 1) < 0.05


def test_streams_are_distinct_and_deterministic():
    a = synth.stream_words(synth.stream_key(1337, 1, 0, 0, 0), 0, 8)
    b = synth.stream_words(synth.stream_key(1337, 1, 0, 1, 0), 0, 8)
    c = synth.stream_words(synth.stream_key(1337, 1, 0, 0, 0), 4, 4)
    assert not np.array_equal(a, b)
    assert np.array_equal(a[4:], c)


def test_zipf_bias_is_a_permutation_of_ranks():
    dims = synth.Dims(4096, 1536, 128, 8, 64)
    b = synth.zipf_bias(1337, dims, 3).astype(np.float64)
    ranks = np.rint(np.exp(-b / 1.1)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, 129))


def test_markov_recursion():
    h = synth.markov_hidden(1337, 3, 64)
    z0 = synth.normal_vector(1337, 0, 64, sub=1)
    z1 = synth.normal_vector(1337, 1, 64, sub=1)
    assert np.allclose(h[0], z0, rtol=1e-6)
    assert np.allclose(h[1], 0.7 * z0 + 0.3 * z1, rtol=1e-5, atol=1e-6)
    # lanes are independent chains
    h5 = synth.markov_hidden(1337, 2, 64, lane=5)
    assert np.allclose(h5[0], synth.normal_vector(1337, 0, 64, sub=6), rtol=1e-6)
    assert not np.allclose(h5[0], h[0])


def test_golden_tiny_decode_reproduces():
    with open(os.path.join(HERE, "golden", "tiny_decode.json")) as f:
        g = json.load(f)
    wl = synth.CONFIGS[0]
    dims = wl.dims
    experts = {e: synth.expert_logical(wl.seed, dims, 0, e) for e in range(dims.n_experts)}
    out = oracle.moe_layer(synth.hidden_bf16(wl.seed, 0, dims.d_model).astype(np.float64),
                           synth.router_bits(wl.seed, dims, 0), experts, dims)
    assert out["idx"] == g["idx"]
    assert [int(b) for b in out["x_bits"]] == g["x_bits"]
    assert np.allclose(out["w"], g["w"], rtol=1e-14)
    assert np.allclose(out["y"], g["y"], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# SMOE-Q2 blobs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wl, blob", [(synth.Q2_WORKLOADS[0], 5898240), (synth.Q2_WORKLOADS[1], 5898240)])
def test_q2_blob_sizes_exact(wl, blob):
    off = synth.blob_sections(wl.dims)
    # codes: 3 * d * f / 4 bytes; params as Q4: 12 * d * f / chunk
    assert off["bytes"] == blob == 3 * 4096 * 1536 // 4 + 12 * 4096 * 1536 // 64
    assert off["stride"] == 360 * 16384
    assert wl.ring_slots in (0, 2764)
    for k, v in off.items():
        assert v % 16 == 0, k
    # the Q4 ring's HBM budget holds 2764 Q2 blobs
    assert 2764 * blob <= 1536 * 10616832 < 2765 * blob


def test_q2_code_and_param_layout():
    dims = synth.Dims(512, 128, 16, 4, 64, bits=2)
    off = synth.blob_sections(dims)
    blob = synth.pack_blob(1337, dims, 0, 3)
    for name, mat, rows, cols in (("gate", 0, 128, 512), ("up", 1, 128, 512), ("down", 2, 512, 128)):
        q = synth.expert_codes(1337, dims, 0, 3, mat)
        sb, mb = synth.expert_params_bits(1337, dims, 0, 3, mat)
        for n, j in ((0, 0), (5, 17), (rows - 1, cols // 4 - 1)):
            byte = int(blob[off[name + "_codes"] + n * cols // 4 + j])
            assert [(byte >> (2 * i)) & 3 for i in range(4)] == q[n, 4 * j:4 * j + 4].tolist()
        nc = cols // dims.chunk
        for n, c in ((0, 0), (7, nc - 1), (rows - 1, 1)):
            p = off[name + "_params"] + (n * nc + c) * 4
            assert int(blob[p]) | int(blob[p + 1]) << 8 == sb[n, c]
            assert int(blob[p + 2]) | int(blob[p + 3]) << 8 == mb[n, c]
    assert np.all(blob[off["bytes"]:] == 0)


def test_q2_packers_agree_and_streams_differ_from_q4():
    dims = synth.Dims(512, 192, 8, 2, 64, bits=2)
    a = synth.pack_blob(7, dims, 2, 5)
    b = synth.pack_logical(dims, synth.expert_logical(7, dims, 2, 5))
    assert np.array_equal(a, b)
    q = np.arange(64, dtype=np.uint8) % 4
    assert np.array_equal(synth.unpack_codes(synth.pack_codes(q, 2), 2), q)
    q4 = synth.expert_codes(7, dims.replace(bits=4), 2, 5, synth.MAT_GATE)
    q2 = synth.expert_codes(7, dims, 2, 5, synth.MAT_GATE)
    assert not np.array_equal(q4 & 3, q2)


def test_q2_distributions():
    dims = synth.Dims(2048, 768, 128, 8, 64, bits=2)
    q = synth.expert_codes(1337, dims, 1, 2, synth.MAT_UP)
    freq = np.bincount(q.reshape(-1), minlength=4) / q.size
    assert np.all(np.abs(freq - 0.25) < 0.002)
    sb, mb = synth.expert_params_bits(1337, dims, 1, 2, synth.MAT_DOWN)
    s, m = oracle.bf16_to_f64(sb), oracle.bf16_to_f64(mb)
    assert s.min() >= 0.002 - 1e-5 and s.max() <= 0.01 + 1e-4
    assert np.array_equal(m, -2 * s)
