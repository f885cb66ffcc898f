"""How far each main-KV format moves the rows and the attention output from the
unquantised bf16 rows, on the synthetic KV distribution (N(0,1) with 1% x20
outliers), measured with the oracle only (CPU).

The pages claim that E4M3 scales per 16 channels keep FP4 accurate enough at
about half the bytes of FP8 ([G], [N]); [T] calls the format MXFP4. The table
below measures that trade on these inputs. Its ordering is asserted: FP8 (4
significant bits per value, 512 B/row) is the most accurate, and the finer,
non-power-of-two E4M3 scale per 16 channels beats MXFP4's power-of-two scale
per 32 channels at almost the same size (288 against 272 B/row).
"""
import numpy as np
import pytest
import torch

from oracle import attention, kvformats
from synth import bf16_to_f64, normal_bf16

FMTS = {"fp4 (E4M3/16)": kvformats.FMT_FP4, "mxfp4 (E8M0/32)": kvformats.FMT_MXFP4, "fp8 (E4M3)": kvformats.FMT_FP8}


def _rel_rms(a, b):
    return float(np.sqrt(np.mean((a - b) ** 2)) / np.sqrt(np.mean(b ** 2)))


def test_format_accuracy_table():
    x = bf16_to_f64(normal_bf16(1, "kv", 0, (4096, 512), outliers=True))
    rng = np.random.default_rng(1)
    q = bf16_to_f64(normal_bf16(1, "q", 0, (4, 64, 512), outliers=False))
    wk = bf16_to_f64(normal_bf16(1, "wk", 0, (4, 128, 512), outliers=False))
    wv = bf16_to_f64(normal_bf16(1, "wv", 0, (4, 128, 512), outliers=False))
    sel = [np.sort(rng.choice(4096, 512, replace=False)) for _ in range(4)]
    scale = 1.0 / np.sqrt(512)
    exact = [attention.attend(q[i], x[sel[i]], wk[i], wv[i], scale)[0] for i in range(4)]
    rows_err, attn_err = {}, {}
    for name, fmt in FMTS.items():
        d = kvformats.dequantize_rows(fmt, *kvformats.quantize_rows(fmt, x))
        rows_err[name] = _rel_rms(d, x)
        errs = []
        for i in range(4):
            o = attention.attend(q[i], d[sel[i]], wk[i], wv[i], scale)[0]
            errs.append(np.abs(o - exact[i]).max() / np.abs(exact[i]).max())
        attn_err[name] = float(max(errs))
    print("\nformat            B/row  rel. RMS row error  max attention error (rel. to max|out|)")
    for name, fmt in FMTS.items():
        print(f"{name:17s} {kvformats.bytes_per_row(fmt, 512):5d}  {rows_err[name]:18.4e}  {attn_err[name]:.4e}")
    f4, mx, f8 = (rows_err[n] for n in FMTS)
    assert f8 < f4 < mx, rows_err
    a4, amx, a8 = (attn_err[n] for n in FMTS)
    assert a8 < a4 < amx, attn_err
