"""Host-side accounting of bench.py (no GPU): the algorithmic bytes and FLOPs
that its roofline figures divide by, checked against counts worked out by hand
from the workload definitions."""
import bench
from synth import workloads as wl


def test_decode128k_scan_bytes():
    # compulsory: 32 queries x 131,072 visible tokens x 256 B of key, plus
    # 16 x 128 x 2 B of query and 16 x 4 B of weights per query
    want = 32 * (131072 * 256 + 16 * 128 * 2 + 16 * 4)
    assert want == 1_073_874_944
    cfg = wl.CONFIGS["decode128k"]
    b = bench.algorithmic_bytes(cfg)
    assert b["scan"] == want
    assert bench.scan_units(cfg) == want
    # intermediates the scan writes for the selection: 4 B per token, 4 B per block
    assert b["scan_intermediate"] == 32 * (131072 * 4 + 16384 * 4) == 18_874_368
    assert bench.scan_intermediate_bytes(cfg) == 18_874_368


def test_decode128k_layer_bytes():
    # per query: keys 33,554,432 + query/weights 4,160 + pool/index lists
    # (2,048 + 512) x 4 + attention 608,256 (512 x 288 B rows, 512 x 4 B indices,
    # Q 64 x 512 bf16, window K and V 2 x 128 x 512 bf16, output 64 x 512 fp32)
    per_q = 33_554_432 + 4_160 + 10_240 + (147_456 + 2_048 + 65_536 + 262_144 + 131_072)
    assert per_q == 34_177_088
    b = bench.algorithmic_bytes(wl.CONFIGS["decode128k"])
    assert b["layer"] == 32 * per_q == 1_093_666_816


def test_prefill_scan_flops():
    # queries at positions 127,000 .. 131,095 see position + 1 tokens each
    pairs = sum(127_000 + i + 1 for i in range(4096))
    assert pairs == 528_582_656
    assert bench.scan_units(wl.CONFIGS["prefill"]) == pairs * 16 * 128 * 2


def test_tiny_and_chain_scan_bytes():
    # one query over 4,096 tokens, indexer 4 x 64: 128 B keys
    assert bench.scan_units(wl.CONFIGS["tiny"]) == 4096 * 128 + 4 * 64 * 2 + 4 * 4
    # eight queries over 2^20 tokens each, indexer 16 x 128
    n = 1 << 20
    assert bench.scan_units(wl.CONFIGS["chain1m"]) == 8 * (n * 256 + 16 * 128 * 2 + 16 * 4)


def test_mixed_scan_bytes_follow_lengths():
    cfg = wl.CONFIGS["mixed"]
    L = cfg.seq_lengths()
    want = sum(int(x) * 256 for x in L) + len(L) * (16 * 128 * 2 + 16 * 4)
    assert bench.scan_units(cfg) == want
    assert all(x % 8 == 0 and 4096 <= x <= 1 << 20 for x in L)


def test_attention_bytes_count_inputs_and_outputs_once():
    cfg = wl.CONFIGS["decode128k"]
    b = bench.algorithmic_bytes(cfg)
    # attention per query: 512 FP4 rows x 288 B, 512 indices, Q 64 x 512 bf16, window K and V
    # 2 x 128 x 512 bf16, output 64 x 512 fp32 and 64 lse
    per_q = 512 * 288 + 512 * 4 + 64 * 512 * 2 + 2 * 128 * 512 * 2 + 64 * 512 * 4 + 64 * 4
    assert b["attn"] == 32 * per_q
    assert b["layer"] < b["scan"] + b["attn"] + b["select"] + b["append"]


def test_kernel_sources_hash_is_stable():
    assert len(bench.sources_hash()) == 16
    assert bench.sources_hash() == bench.sources_hash()


def test_kernel_sources_cover_every_source_file():
    # the hash that dates the stored counter traffic must change with any kernel source
    import os
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "sparse_indexer_fp4_amd", "csrc")
    on_disk = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    assert sorted(bench.KERNEL_SOURCES) == on_disk


def test_inputs_hash_covers_names_shapes_bytes_and_order():
    """The input digest is SHA-256 over (name, dtype, shape) headers and the raw
    bytes, in order; a changed byte, shape, name or order changes it, and a
    missing (None) tensor is skipped. Tensors larger than one 64 MiB piece are
    hashed piece by piece to the same digest."""
    import hashlib
    import torch
    x = torch.arange(10, dtype=torch.bfloat16)
    y = torch.arange(6, dtype=torch.int64).reshape(2, 3)
    h = hashlib.sha256()
    h.update(b"x:torch.bfloat16:(10,);")
    h.update(x.view(torch.uint8).numpy().tobytes())
    h.update(b"y:torch.int64:(2, 3);")
    h.update(y.reshape(-1).view(torch.uint8).numpy().tobytes())
    base = bench.inputs_sha256([("x", x), ("gone", None), ("y", y)])
    assert base == h.hexdigest()[:16]
    x2 = x.clone()
    x2[3] = 100.0
    assert bench.inputs_sha256([("x", x2), ("y", y)]) != base
    assert bench.inputs_sha256([("x", x), ("y", y.reshape(3, 2))]) != base
    assert bench.inputs_sha256([("x", x), ("z", y)]) != base
    assert bench.inputs_sha256([("y", y), ("x", x)]) != base
    big = torch.arange((64 << 20) // 4 + 5, dtype=torch.int32)
    hb = hashlib.sha256()
    hb.update(f"big:torch.int32:{tuple(big.shape)};".encode())
    hb.update(big.numpy().tobytes())
    assert bench.inputs_sha256([("big", big)]) == hb.hexdigest()[:16]
