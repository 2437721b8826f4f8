"""The algorithmic bytes and flops behind every roofline figure the benchmark prints, worked
out by hand from the decode workload's shapes (B=32, 64K context, 64 indexer heads x 128
dims, 128 MLA heads over 576-wide latent rows, top-2048, 64-token pages)."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_decode_step_work():
    w = _bench().algorithmic_work(32, 65536, 64, 128, 2048, 128, 64)
    keys = 32 * 65536 * 128                   # e4m3 codes
    sigma = 32 * 65536 * 4                    # one float32 scale per token
    q = 32 * 64 * 128 * 2                     # bf16 queries
    wts = 32 * 64 * 4                         # head weights
    pages = 32 * 1024 * 4                     # page table
    scores = 32 * 65536 * 4                   # float32 scores out
    assert w["indexer"] == (keys + sigma + q + wts + pages + scores, 2 * 32 * 64 * 128 * 65536)
    assert w["indexer"][0] == 285_876_224
    assert w["topk"] == (scores + 32 * 2048 * 4, 0)
    # with the chunk stage in the scan's epilogue the top-k stage only writes the indices
    wf = _bench().algorithmic_work(32, 65536, 64, 128, 2048, 128, 64, topk_fused=True)
    assert wf["topk"] == (32 * 2048 * 4, 0) and wf["indexer"] == w["indexer"] and wf["mla"] == w["mla"]
    rows = 32 * 2048 * 1152                   # selected 576-wide bf16 latent rows
    mla_q, idx, o, lse = 32 * 128 * 576 * 2, 32 * 2048 * 4, 32 * 128 * 512 * 2, 32 * 128 * 4
    assert w["mla"] == (rows + mla_q + idx + o + lse, 2 * 32 * 128 * 2048 * (576 + 512))
    assert w["mla"][0] == 84_688_896


def test_fp4_cache_and_mtp_work():
    b = _bench()
    w = b.algorithmic_work(32, 65536, 64, 128, 2048, 128, 64, keys="mxfp4")
    # 64 bytes of E2M1 codes + 4 E8M0 scales per token replace 128 + 4
    assert w["indexer"][0] == 285_876_224 - 32 * 65536 * (132 - 68)
    assert w["indexer"][0] == 151_658_496
    # MTP verify: keys read once for the four queries, everything per query scales by four
    m = b.algorithmic_work(8, 200004, 64, 128, 2048, 128, 64, Sq=4, q_bytes=1)
    assert m["indexer"][1] == 2 * 32 * 64 * 128 * 200004
    assert m["indexer"][0] == (8 * 200004 * 132 + 32 * 64 * 128 + 32 * 64 * 4 + 8 * 3126 * 4
                               + 32 * 200004 * 4)
