"""CPU oracle for the HiSparse decode path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct reimplementation of what the decode path
computes, written from the pages that describe HiSparse:

* the HiSparse summary article ("显存占用直降30倍！大模型稀疏注意力解码KV缓存
  方案HiSparse夯爆了"), section 02: full KV lives in pinned host memory, a
  fixed B-slot device buffer per request and layer caches recently selected
  rows, a page table maps logical positions to slots or "host only", LRU
  metadata drives replacement, RESOLVE fuses hit detection, replacement,
  metadata update and the host fetch, and the method is exact (only the
  placement of KV changes, not scores or outputs);
* the vLLM blog "GLM 5.3 优化（一）：vLLM 的 Hybrid HiSparse 混合稀疏卸载",
  section "工作原理" (how it works): mixed residency, where GPU-resident pages
  are read in place, hot tokens are read and their LRU entry refreshed, and a
  miss copies a single row from pinned host memory into an LRU slot; the tail
  page is never evicted.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this package.  It shares no code with the HIP library or its
Python binding, and imports only ``tracegen`` (the seeded input generator).

Modules:
  resolve     exact step-LRU RESOLVE (the state machine)
  bruteforce  an independent per-miss scan replay of the same rules (a pin)
  textbook    a textbook LRU cache (OrderedDict), for the K=1 reduction pin
  attention   dense fp64 softmax attention over the selected rows
  step        one decode step over a workload (resolve every layer of a
              group, then attend every layer)
  prefetch    cross-step prefetch of a predicted selection into the buffer
"""
