"""CSA2 layer schedules through the C ABI: the 4,096-query prefill chunk through
a Full group and a Reindex group (F R R R, Ri R R R), the 20 decoder layers
(F R R R, then 4 x Ri R R R) at 1M context, and the 18 encoder layers
(3 x F R R R R R) over a 1,024-query chunk.

Sampled queries are recomputed layer by layer by the oracle's schedule (the
indices each layer attends with) from host-regenerated inputs: pools and
indices bit-exact, attention within max|out - ref| <= 2e-4 * max|ref| + 1e-6.
Each schedule then runs a second time and prints its per-layer times.
"""
import numpy as np
import pytest
import torch

from oracle import chain
from synth import workloads as wl
from tests import oracle_runner as orun
from tests.schedule_runner import run_schedule, timing_table

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_indexer_fp4_amd as m
    return m


def _say(msg):
    print(msg, flush=True)


def _check(cfg, layers, queries, k_rows_of):
    for i in queries:
        k_rows = k_rows_of(i)
        ref = chain.layer_indices(
            cfg.modes,
            lambda layer: orun.full_layer(cfg, i, layer, k_rows=k_rows)[:2],
            lambda layer, pool: orun.reindex_layer(cfg, i, layer, pool))
        for layer, rec in enumerate(layers):
            rp, ri = ref[layer]
            if rec["mode"] == "full":
                n_pool = int(rec["n_pool"][i])
                got_pool = rec["pool"][i].cpu().numpy()
                assert n_pool == len(rp) and np.array_equal(got_pool[:n_pool], rp), (i, layer)
            n = int(rec["n_idx"][i])
            got = rec["idx"][i].cpu().numpy()
            assert n == len(ri) and np.array_equal(got[:n], ri) and (got[n:] == -1).all(), (i, layer)
            ro, rl = orun.attend(cfg, i, layer, ri)
            ok, err, tol = orun.within_tolerance(rec["out"][i].cpu().numpy(), ro)
            assert ok, ("out", i, layer, err, tol)
            ok, err, tol = orun.within_tolerance(rec["lse"][i].cpu().numpy(), rl)
            assert ok, ("lse", i, layer, err, tol)
        _say(f"{cfg.name}: query {i} matches the oracle on all {len(layers)} layers")


def _run(fk, name, queries, per_query_rows):
    from tests.gpu_inputs import DeviceWorkload
    cfg = wl.CONFIGS[name]
    _say(f"{name}: setup")
    dw = DeviceWorkload(cfg, torch.device("cuda"))
    layers = run_schedule(fk, cfg, dw)
    _say(f"{name}: checking")
    shared = None if per_query_rows else orun.host_idx_k(cfg, 0, cfg.ctx)
    k_rows_of = (lambda i: orun.host_idx_k(cfg, wl.sequence_of(cfg, i), int(cfg.q_pos()[i]) + 1)) \
        if per_query_rows else (lambda i: shared)
    _check(cfg, layers, queries, k_rows_of)
    del layers
    torch.cuda.empty_cache()
    _say(timing_table(cfg, run_schedule(fk, cfg, dw)))


def test_prefill_full_and_reindex_groups(fk):
    """The prefill chunk through F R R R, then Ri R R R on the Full layer's pool."""
    _run(fk, "prefill_chain", (0, 2048, 4095), per_query_rows=False)


def test_decoder_schedule_1m(fk):
    """The 20 decoder layers at 1M context for 4 queries."""
    _run(fk, "decoder1m", (0, 3), per_query_rows=True)


def test_encoder_schedule(fk):
    """The 18 encoder layers over a 1,024-query chunk (three Full groups)."""
    _run(fk, "encoder_chunk", (0, 1023), per_query_rows=False)
