"""Plain, slow CPU oracle for the CSA2 sparse-attention hot path (float64 numpy).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import it: only the
tests, the smoke check and the benchmark's CPU-baseline leg call it. It shares
no code with the HIP library and does not import it.

Sources (web pages on DeepSeek V4.1-Flash's KV cache):
  [G]  "DeepSeek V4.1 Flash KV Cache: 890 Bytes per Token Explained"
       (deepseekv4guide.org; the page has no section headings, so a paragraph
       topic is named instead: "CSA2 modes", "hierarchical sparse indexer",
       "FP4 main KV", "SWA Bounded Replay").
  [T]  "890 bytes per token: how DeepSeek V4.1-Flash's KV cache works"
       (runaii.cloud), sections "Mechanism 3: FP4 KV via quantization-aware
       training" and "Mechanism 4: the hierarchical sparse indexer".
  [N]  "DeepSeek-V4.1-Flash: 890 Bytes Per Token, 437x Smaller KV Cache"
       (aimastery.page), sections "CSA2: Sharing Main KV, Indexer K, and Top-K
       Indices Across Layers", "FP4 KV Quantization and Cache Lifetime
       Management" and "Causal Encoder-Decoder and Prefill Halving".

The pages name the mechanisms but leave the scoring rule, tie-breaks, rounding
and attention details open. The readings taken here:
  * indexer score of token t: sum over heads h of w_h * max(0, q_h . k_t), one
    indexer key per token shared by all heads;
  * block score: max over the block's visible tokens (blocks of 8 from
    position 0); visible means position <= the query's position;
  * ranking: score descending, then position ascending (lower index wins a
    tie); results are returned in ascending position;
  * scale: E4M3 value nearest amax/6, ties to the even code, saturating at
    448; values: E2M1 value nearest |x|/scale, ties to the even code,
    saturating at 6; sign bit copied from x; scale 0 gives magnitude 0;
  * attention: keys = values = the dequantised row (MQA latent); the window
    branch covers positions max(0, p-127)..p; branches merge by log-sum-exp.

Modules: fp4 (codec), indexer (scores, blocks, selection, Full/Reindex),
attention (branches and merge), chain (Full/Reindex/Reuse schedule).

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_*.py (closed forms, library routines, brute force on tiny
inputs, worked examples under tests/golden/, and invariants).
"""
from . import fp4, indexer, attention, chain  # noqa: F401
