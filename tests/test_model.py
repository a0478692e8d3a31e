"""The alpha-beta module against the numbers the pages print (CPU only)."""

import json
import os

import pytest

from collective_communication_algorithms_amd import model

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "alpha_beta_tables.json")))


def test_allreduce_comparison_table_n8():
    t = G["allreduce_compare_n8"]
    for algo in ("ring", "rhd", "dbt"):
        assert model.latency_steps("allreduce", algo, 8) == t[algo]["latency_alpha"]
        assert model.bandwidth_coef("allreduce", algo, 8) == pytest.approx(t[algo]["bw_coef"])


def test_latency_terms_at_large_n():
    assert model.latency_steps("allreduce", "ring", 8) == G["ring_latency_terms"]["n8_alpha"]
    assert model.latency_steps("allreduce", "ring", 1024) == G["ring_latency_terms"]["n1024_alpha"]
    assert model.latency_steps("allreduce", "rhd", 64) == G["rhd_vs_ring_n64"]["rhd_alpha"]
    assert model.latency_steps("allreduce", "ring", 64) == G["rhd_vs_ring_n64"]["ring_alpha"]


def test_ring_dbt_crossover():
    c = G["ring_dbt_crossover"]
    m = model.ring_dbt_crossover(c["nranks"], c["alpha_us"] * 1e-6, c["beta_GBps"] * 1e9)
    assert m / 1e6 == pytest.approx(c["M_star_MB"], rel=1e-3)
    # at the crossover the two formulas agree
    a, b = c["alpha_us"] * 1e-6, c["beta_GBps"] * 1e9
    assert model.time("allreduce", "ring", 8, m, a, b) == pytest.approx(model.time("allreduce", "dbt", 8, m, a, b))


@pytest.mark.parametrize("N", [2, 4, 8, 16, 64])
def test_busbw_coefficients(N):
    t = G["busbw_coefficients"]
    import re
    env = {"N": N}
    for kind in ("allreduce", "allgather", "reducescatter", "alltoall", "broadcast", "reduce"):
        expr = re.sub(r"(\d)\(", r"\1*(", t[kind])        # the table writes 2(N-1)/N
        assert model.busbw_coef(kind, N) == pytest.approx(eval(expr, {}, env))


@pytest.mark.parametrize("N", [2, 3, 8, 13, 64])
def test_ring_identity(N):
    """T_Ring-AR = T_Ring-RS + T_Ring-AG."""
    a, b, M = 5e-6, 450e9, 1 << 24
    assert model.time("allreduce", "ring", N, M, a, b) == pytest.approx(
        model.time("reducescatter", "ring", N, M, a, b) + model.time("allgather", "ring", N, M, a, b))


def test_pipelines_reduce_to_their_k1_forms():
    a, b, M = 5e-6, 450e9, 1 << 20
    assert model.time("broadcast", "chain_pipe", 8, M, a, b, 1) == pytest.approx(model.time("broadcast", "chain", 8, M, a, b))
    assert model.time("broadcast", "binomial_pipe", 8, M, a, b, 1) == pytest.approx(model.time("broadcast", "binomial", 8, M, a, b))


def test_best_chunks_is_the_argmin_of_the_formula():
    a, b = 5e-6, 450e9
    got = [model.best_chunks("chain_pipe", 8, m, a, b) for m in (1024, 65536, 4 << 20, 64 << 20)]
    assert got == [1, 1, 3, 13]
    got = [model.best_chunks("binomial_pipe", 8, m, a, b) for m in (1024, 65536, 4 << 20, 64 << 20)]
    assert got == [1, 1, 2, 8]
    for m in (1024, 4 << 20, 64 << 20):
        k = model.best_chunks("chain_pipe", 8, m, a, b)
        t = model.time("broadcast", "chain_pipe", 8, m, a, b, k)
        assert all(model.time("broadcast", "chain_pipe", 8, m, a, b, j) >= t for j in range(1, 200))


def test_reduce_and_scatter_formulas():
    """Tree Reduce has the tree Broadcast's formula (eq:model-algo-reduce-tree);
    naive Scatter is (N-1)(alpha + M/(N beta)) (eq:onetoall-scatter-naive)."""
    a, b, M = 5e-6, 450e9, 1 << 24
    for N in (2, 8, 16):
        assert model.time("reduce", "binomial", N, M, a, b) == pytest.approx(model.time("broadcast", "binomial", N, M, a, b))
        assert model.time("scatter", "linear", N, M, a, b) == pytest.approx((N - 1) * (a + M / (N * b)))
        assert model.latency_steps("broadcast", "scatter_allgather", N) == (N - 1) + model.latency_steps("scatter", "binomial", N)


def test_bidir_ring_broadcast_formula():
    """The 4-chip bidirectional ring takes 2 iterations, the ceil(log2 N) lower
    bound ("SCCL 的 Broadcast 实现"); in general the half-ring chain is
    ceil((N-1)/2) hops, pipelined like eq:pipe-chain-bcast."""
    a, b, M = 5e-6, 450e9, 1 << 22
    assert model.latency_steps("broadcast", "bidir_ring", 4) == 2
    for N in (2, 3, 5, 8, 9):
        for k in (1, 4):
            h = (N - 1 + 1) // 2
            assert model.time("broadcast", "bidir_ring", N, M, a, b, k) == pytest.approx((h + k - 1) * (a + M / (k * b)))
    # with N - 1 ranks past the root in one direction it would be the chain pipeline
    assert model.time("broadcast", "bidir_ring", 8, M, a, b, 4) < model.time("broadcast", "chain_pipe", 8, M, a, b, 4)


def test_overlap_estimate_matches_printed_examples():
    """The blog prints the estimate for ResNet-50 (150 / 50 ms) and BERT-Large
    (100 / 80 ms); its prose elsewhere gives other figures (a contradiction
    inside the page), the printed function's outputs are the pin."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "overlap_examples.json")))
    for ex in g["examples"]:
        assert model.serial_time(ex["compute_ms"], ex["comm_ms"]) == ex["no_overlap_ms"]
        assert model.overlapped_time(ex["compute_ms"], ex["comm_ms"]) == ex["overlap_ms"]


def test_hidden_fraction_limits():
    assert model.hidden_fraction(100, 50, 100) == 1.0      # fully hidden
    assert model.hidden_fraction(100, 50, 150) == 0.0      # serialised
    assert model.hidden_fraction(30, 50, 50) == pytest.approx(0.6)
