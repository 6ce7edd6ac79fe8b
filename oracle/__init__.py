"""Oracle: a plain, slow, fp64 CPU statement of what the sliding-window attention path computes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package may import, call or link anything
here; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code, tables or constants with the HIP library: it knows positions, keys
and values only, never the device pool layout.

Sources (web pages; cited by page title and section, equation or table):

* [SWA-theory] disassemble-channel.com, "Sliding Window Attention（SWA）の理論と実装 —
  固定窓による局所注意とMistralでの採用": the window W(i) (§数学的定義, Eq.(1)), the mask
  (Eq.(2)), the masked score (Eq.(3)), softmax (Eq.(4)), the output sum (Eq.(5)), the scaled
  dot-product attention formula (§Full Attentionの問題点), the receptive field (§窓サイズと有効受容野,
  Eq.(6)), GQA sharing (§MistralにおけるSWAの採用), the rolling buffer slot rule
  (§Rolling Buffer KV Cache, Eq.(7)) and the KV size calculator (§計算時間・メモリ比較実験).
* [MiMo-review] youngju.dev review of Xiaomi's MiMo-V2.5 inference post: the 60 SWA / 10 full
  hybrid stack with w=128 (§アーキテクチャ), the KV ratio (60·W+10·N)/(70·N) (same section), the
  dual pool and the window-safe prefix length (§潜在力を本番へ), and FP8 storage of the windowed
  cache as the orthogonal axis (§おわりに).
* The E4M3 format itself is the OCP 8-bit floating point specification's (OFP8).
* RoPE, which [SWA-theory] §Rolling Buffer KV Cache relies on without writing it out, is the
  published RoFormer definition (Su et al., 2021, §3.2-§3.4).

Modules
-------
``oracle.attention``  Eq.(1)-(5): key sets, masks, fp64 two-pass softmax attention by position.
``oracle.kvcache``    Eq.(7) rolling buffer model, paged placement, window-safe length (brute force
                      and closed form), KV byte accounting, hybrid layer map, receptive field.
``oracle.fp8``        E4M3 encode (nearest, ties to even, saturating) / decode and the per-pool
                      power-of-two scale of FP8 KV storage.
``oracle.rope``       rotary position embedding of queries and keys (pairs or split-halves layout).

Every function is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_pins.py`` against
values the pages print, closed forms, library routines (torch SDPA in float64, torch's
float8_e4m3fn conversion, numpy complex exponentials) or brute force.
No function here is "parity unpinned".
"""
