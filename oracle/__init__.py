"""fp64 CPU oracle for SegPagedAttention prefill -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The library path never calls it, and it never calls the library:
the two share no code.  Everything here is plain, slow and written to be checked
against the pages by eye.

Sources (web pages about RedKnot; cited by title and section):
  [ZC] "小红书把 KV Cache 按「头」拆了——长文本推理的「稠密时代」可能正在结束" (zhichai.net)
  [SS] "RedKnot – 小红书研发并开源的长上下文大模型推理引擎" (shshi.cn)
  [BJ] "为什么长上下文推理这么慢？RedKnot如何用1个百分点的质量代价换来2–5倍TTFT加速" (bjdmk.com.cn)
  [AB] "RedKnot - Xiaohongshuが開発したオープンソースの長文テキスト推論高速化エンジン" (aiboss88.com)

Modules:
  attention -- visibility mask per head class and dense masked softmax attention in fp64
  rope      -- rotary re-rotation of reused keys from their offline to their actual position
  paging    -- held token ranges, page sets, allocator replay, visible intervals, pair counts
  reference -- one prefill call of a synthetic workload, assembled from the three above

Every function is pinned by a `-m "not gpu"` test against something other than
itself (closed forms, library routines, brute force, hand-derived fixtures).
"""
