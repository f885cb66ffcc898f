"""The allocation-free Full indexer (fp4kv_index_full_noalloc) against
fp4kv_index_full, through the C ABI: identical pools and indices, bit for bit,
on two calls in a row, the second one smaller (so the fixed device workspace
still holds the first call's scores), for the per-query scan and for the
matrix-core scan of many queries per sequence; calls beyond the fixed size are
refused before anything runs."""
import numpy as np
import pytest
import torch

from synth import int_tensor_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import sparse_indexer_fp4_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return m


def _say(msg):
    print(msg, flush=True)


def _inputs(gpu, lengths, H, D, seed, q_per_seq=1, positions=None):
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    total = int(np.sum(lengths))
    kk = int_tensor_bf16(seed, "k", 0, (total, D), -8, 8, device=gpu)
    qpos = (np.asarray(lengths) - 1) if positions is None else np.asarray(positions)
    nq = len(qpos)
    q = int_tensor_bf16(seed, "q", 0, (nq, H, D), -8, 8, device=gpu)
    w = torch.randint(1, 9, (nq, H), generator=torch.Generator().manual_seed(seed)).to(torch.float32).to(gpu)
    return (q, w, kk, torch.from_numpy(starts).to(gpu), torch.from_numpy(qpos.astype(np.int32)).to(gpu),
            int(qpos.max()) + 1)


def _compare(fk, gpu, args, q_per_seq, P, k):
    q, w, kk, starts, qpos, max_ctx = args
    nq = q.shape[0]
    ref = fk.fp4kv_index_full(q, w, kk, starts, qpos, q_per_seq, max_ctx, P, k)
    outs = [torch.full((nq, P), -7, dtype=torch.int32, device=gpu), torch.full((nq,), -7, dtype=torch.int32, device=gpu),
            torch.full((nq, k), -7, dtype=torch.int32, device=gpu), torch.full((nq,), -7, dtype=torch.int32, device=gpu)]
    got = fk.fp4kv_index_full_noalloc(q, w, kk, starts, qpos, q_per_seq, max_ctx, P, k, *outs)
    torch.cuda.synchronize()
    for name, a, b in zip(("pool", "n_pool", "idx", "n_idx"), ref, got):
        assert torch.equal(a, b), name
    assert int(got[3].min()) > 0


def test_noalloc_matches_index_full_two_calls(fk, gpu):
    _say("index_full_noalloc: per-query scan, large then small call")
    _compare(fk, gpu, _inputs(gpu, [60000, 131072, 777, 45001, 90000, 8], 16, 128, seed=71), 1, 2048, 512)
    _compare(fk, gpu, _inputs(gpu, [5000, 3, 12345], 16, 128, seed=72), 1, 64, 100)


def test_noalloc_matches_index_full_many_queries_per_sequence(fk, gpu):
    _say("index_full_noalloc: matrix-core scan, large then small call")
    L = 20000
    _compare(fk, gpu, _inputs(gpu, [L], 16, 128, seed=73, positions=list(range(L - 96, L))), 96, 512, 256)
    L = 3000
    _compare(fk, gpu, _inputs(gpu, [L], 16, 128, seed=74, positions=list(range(L - 32, L))), 32, 16, 40)


def test_noalloc_refuses_calls_beyond_its_workspace(fk, gpu):
    _say("index_full_noalloc: size limit")
    q, w, kk, starts, qpos, _ = _inputs(gpu, [100, 100], 16, 128, seed=75)
    outs = [torch.empty((2, 64), dtype=torch.int32, device=gpu), torch.empty((2,), dtype=torch.int32, device=gpu),
            torch.empty((2, 64), dtype=torch.int32, device=gpu), torch.empty((2,), dtype=torch.int32, device=gpu)]
    with pytest.raises(fk.Fp4kvError) as e:
        fk.fp4kv_index_full_noalloc(q, w, kk, starts, qpos, 1, 1 << 23, 64, 64, *outs)
    assert e.value.status == -3
