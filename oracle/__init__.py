"""CPU oracle for the DSA sparse-attention decode step — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, single-threaded restatement of what the decode step
computes, in float64 where it computes in floating point.  It exists to check the
HIP library, and nothing on the product path may import, call or link it: only the
test-suite, the smoke check and the CPU-baseline leg of the benchmark use it.  It
shares no code with the HIP path; it reads the same seeded input bytes.

Sources (web pages the method is described on):
  [GLM52]  "Shared-Indexer KV Cache Offload for GLM-5.2 on CANN" (lmnt.cn news 268566)
  [HCCP]   "HiCache across parallel modes and distributed serving" (dujian.net)
  [TSA]    TokenSpeed engine code audit (devpress.csdn.net, AMD channel)
  [GLM5R]  Zhipu GLM-5 serving report (hkstock.com.hk news 808716)

Functions and what pins them (tests/test_oracle_*.py):
  formats.bf16_to_f64 / e4m3_to_f64     torch's own bf16 / float8_e4m3fn decoders, all codes
  paging.owner_local                    brute-force page enumeration; [HCCP] §1.1 worked example
  indexer.scores                        integer-exact grid cross-check, single-head dot product,
                                        ReLU/weight/scale special cases
  topk.select                           full sort vs heapq.nlargest; brute force; tie/sign cases
  plan.plan_step                        deque-per-set FIFO simulator; invariants; special cases
  gather.gather_rows / install          byte equality with the cache; pool == cache at live slots
  mla.sparse_mla / lse_merge            dense softmax attention (torch SDPA in float64) when
                                        every token is selected; one-row and permutation cases;
                                        merge over any partition == attention over the union
"""
from . import formats, paging, indexer, topk, plan, gather, mla, step  # noqa: F401
