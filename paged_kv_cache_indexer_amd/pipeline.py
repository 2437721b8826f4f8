"""Orchestration of libdsa's entry points into decode steps: plumbing only.

Every stage runs in libdsa's kernels; this module owns the device buffers a step reuses
(so a step can be captured into a HIP graph and replayed) and the order and streams the
entry points are enqueued on.

  DecodeStep     indexer scan -> top-k -> sparse MLA over the paged latent cache, the
                 decode path of the GLM-5.2 shared-Indexer page (§2.1), with per-layer
                 caches that successive calls rotate through
  PoolGroupStep  one decode step of a shared-indexer group (§4.1: groups of 4 layers share
                 one top-k): one plan (§4.2-4.3), then per layer serve -> attention ->
                 install (§4.4), installs optionally on an auxiliary stream
  MtpDraftSteps  MTP draft steps over a frozen selection (§5.1): the first serve's
                 selection buffer is reused by the later draft steps
  HipMark        a HIP timing event on a given stream (torch's events only see torch's
                 current stream)
"""
import ctypes
from dataclasses import dataclass
from typing import List, Optional

import torch

from . import _lib, api as dsa

_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventRecordWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    return _hip


class HipMark:
    """A HIP timing event recorded on a stream; `external=True` records it as an external
    event node when the stream is being captured into a graph."""

    def __init__(self, external: bool = False):
        hip = _hiprt()
        self.ev = ctypes.c_void_p()
        rc = hip.hipEventCreate(ctypes.byref(self.ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.flags = 1 if external else 0          # hipEventRecordExternal

    def record(self, stream):
        rc = _hiprt().hipEventRecordWithFlags(self.ev, stream.cuda_stream, self.flags)
        if rc != 0:
            raise RuntimeError(f"hipEventRecordWithFlags failed ({rc})")

    def elapsed_ms(self, end: "HipMark") -> float:
        ms = ctypes.c_float()
        rc = _hiprt().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value


def host_device_ptr(t: torch.Tensor) -> int:
    """Device alias of a pinned host tensor (hipHostGetDevicePointer)."""
    dptr = ctypes.c_void_p()
    rc = _hiprt().hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
    if rc != 0:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({rc})")
    return dptr.value


@dataclass
class LayerCaches:
    """One layer's caches: indexer keys (row store, per-token scale or MXFP4 block scales)
    and latent rows."""
    keys: dsa.Rows
    k_scale: Optional[torch.Tensor]
    kv: dsa.Rows


class DecodeStep:
    """One decode step (indexer -> top-k -> sparse MLA) over fixed device buffers.

    All buffers are allocated once, so the step can be captured into a HIP graph and
    replayed.  `run(stream, marks, layer)` enqueues the three stages on `stream`, reading the
    caches of layer `layer % len(layers)` (successive layers of a model read different
    caches).  `marks`, if given, are four objects with a `record(stream)` method, recorded
    before, between and after the stages.

    With `fused` (the default), a step with one query token per request runs the top-k's
    chunk stage inside the scan (dsa_indexer_topk_chunks, then dsa_topk_select_chunks);
    shapes the fused entry points do not take (it rejects them before enqueuing anything)
    fall back to dsa_indexer_scores and dsa_topk.  Both give identical results.
    """

    def __init__(self, idx_q: torch.Tensor, idx_w: torch.Tensor, seq_lens: torch.Tensor, mla_q: torch.Tensor,
                 layers: List[LayerCaches], topk: int, scale: float, max_len: int, k_dtype: int, q_dtype: int,
                 err: Optional[torch.Tensor] = None, o_dtype=torch.bfloat16, fused: bool = True):
        dev = idx_q.device
        self.fused = None if fused else False     # None: not tried yet
        self.topk, self.max_len, self.o_dtype = topk, max_len, o_dtype
        self.idx_q, self.idx_w, self.seq_lens, self.mla_q = idx_q, idx_w, seq_lens, mla_q
        self.layers, self.scale, self.k_dtype, self.q_dtype = layers, scale, k_dtype, q_dtype
        self.err = err if err is not None else torch.zeros(1, dtype=torch.int32, device=dev)
        B, Sq = idx_q.shape[:2]
        H = mla_q.shape[2]
        self.scores = torch.empty((B, Sq, max_len), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B, Sq, topk), dtype=torch.int32, device=dev)
        self.o = torch.empty((B, Sq, H, 512), dtype=o_dtype, device=dev)
        self.lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)
        self.ws_mla = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(B, Sq, H, topk)), dtype=torch.uint8,
                                  device=dev)
        self.ws_topk = torch.empty(max(1, dsa.dsa_topk_workspace_size(B, Sq, topk, max_len)), dtype=torch.uint8,
                                   device=dev)

    def with_form(self, fused: bool) -> "DecodeStep":
        """A step over the same inputs and layer caches (own outputs and workspaces) that
        takes the fused or the separate scan and top-k."""
        return DecodeStep(self.idx_q, self.idx_w, self.seq_lens, self.mla_q, self.layers, self.topk, self.scale,
                          self.max_len, self.k_dtype, self.q_dtype, err=self.err, o_dtype=self.o_dtype, fused=fused)

    def stage(self, name, stream, layer=0):
        """Enqueue one stage ("indexer", "topk" or "mla") of the step on `stream`."""
        lc = self.layers[layer % len(self.layers)]
        if name == "indexer":
            if self.fused is not False and self.idx.shape[1] == 1:
                try:
                    dsa.dsa_indexer_topk_chunks(self.idx_q, self.idx_w, lc.keys, lc.k_scale, self.seq_lens,
                                                self.scores, self.idx.shape[-1], self.ws_topk, k_dtype=self.k_dtype,
                                                err=self.err, q_dtype=self.q_dtype, stream=stream)
                    self.fused = True
                    return
                except dsa.DsaError as e:
                    if self.fused or e.status != _lib.DSA_ERR_UNSUPPORTED:
                        raise
            self.fused = False
            dsa.dsa_indexer_scores(self.idx_q, self.idx_w, lc.keys, lc.k_scale, self.seq_lens, self.scores,
                                   k_dtype=self.k_dtype, err=self.err, q_dtype=self.q_dtype, stream=stream)
        elif name == "topk":
            if self.fused:
                dsa.dsa_topk_select_chunks(self.scores, self.seq_lens, self.idx, self.ws_topk, stream=stream)
            else:
                dsa.dsa_topk(self.scores, self.seq_lens, self.idx, ws=self.ws_topk, stream=stream)
        elif name == "mla":
            dsa.dsa_sparse_mla_decode(self.mla_q, self.idx, lc.kv, self.scale, self.o, self.lse, ws=self.ws_mla,
                                      err=self.err, stream=stream)
        else:
            raise ValueError(name)

    def run(self, stream, marks=None, layer=0):
        for j, name in enumerate(("indexer", "topk", "mla")):
            if marks:
                marks[j].record(stream)
            self.stage(name, stream, layer)
        if marks:
            marks[3].record(stream)


class PoolGroupStep:
    """One decode step of the device-pool workload for the layers of one shared group:
    one plan (committed at plan time), then per layer serve -> attention -> install.

    Serve writes each layer's selection buffer and its index list (entry j, or -1 where a
    padding entry got the zero row), and attention reads the buffer through that list, so
    padding never enters the softmax.

    With `aux_install`, each layer's install runs on a second stream: it waits for that
    layer's serve (it reads the served rows) and overlaps the layer's attention, and the
    next step's serve of the layer waits for it (it reads pool rows the install writes and
    overwrites the served rows the install reads).  The plan outputs alternate between two
    buffers, so the next step's plan never overwrites what a pending install still reads.

    host : list (one per layer) of Rows over the request-major host rows [B*L, 576]
    """

    def __init__(self, B, k, H, n_sets, ways, id_range, host, scale, aux_install=False, device="cuda"):
        self.B, self.k, self.H, self.S, self.W, self.idr = B, k, H, n_sets, ways, id_range
        self.host, self.scale, self.aux = host, scale, aux_install
        self.layers = len(host)
        dev = device
        self.pool = [torch.zeros((B, n_sets * ways, 576), dtype=torch.bfloat16, device=dev) for _ in host]
        self.sel = [torch.empty((B, 1, k, 576), dtype=torch.bfloat16, device=dev) for _ in host]
        self.sel_idx = [torch.empty((B, 1, k), dtype=torch.int32, device=dev) for _ in host]
        self.sel_rows = [dsa.Rows(s, 1152, req_stride=k) for s in self.sel]
        self.o = [torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=dev) for _ in host]
        self.lse = [torch.empty((B, 1, H), dtype=torch.float32, device=dev) for _ in host]
        self.pids = torch.full((B, n_sets * ways), -1, dtype=torch.int32, device=dev)
        self.its = torch.full((B, id_range), -1, dtype=torch.int32, device=dev)
        self.ptr = torch.zeros((B, n_sets), dtype=torch.int32, device=dev)
        self.plan_out = [dict(is_hit=torch.empty((B, 1, k), dtype=torch.uint8, device=dev),
                              slot=torch.empty((B, 1, k), dtype=torch.int32, device=dev),
                              mp=torch.empty((B, k), dtype=torch.int32, device=dev),
                              ms=torch.empty((B, k), dtype=torch.int32, device=dev),
                              mc=torch.empty(B, dtype=torch.int32, device=dev)) for _ in range(2)]
        self.ws = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(B, 1, H, k)), dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.aux_stream = torch.cuda.Stream() if aux_install else None
        self.installed = [torch.cuda.Event() for _ in host]          # layer l's last install
        self.plan_free = [torch.cuda.Event() for _ in range(2)]      # installs of the buffer's last step
        self.step_no = 0

    def plan(self, stream, topk, po):
        dsa.dsa_plan(topk, self.pids, self.its, self.ptr, self.S, self.W, po["is_hit"], po["slot"], po["mp"],
                     po["ms"], po["mc"], commit=True, err=self.err, stream=stream)

    def serve(self, stream, topk, po, l):
        dsa.dsa_gather_kv(topk, po["is_hit"], po["slot"], self.host[l], self.pool[l], self.sel[l],
                          dsa.DSA_GATHER_SERVE, err=self.err, stream=stream, sel_idx=self.sel_idx[l])

    def attend(self, stream, q, l):
        dsa.dsa_sparse_mla_decode(q, self.sel_idx[l], self.sel_rows[l], self.scale, self.o[l], self.lse[l],
                                  ws=self.ws, err=self.err, stream=stream)

    def install(self, stream, topk, po, l):
        dsa.dsa_gather_kv(topk, po["is_hit"], po["slot"], None, self.pool[l], self.sel[l],
                          dsa.DSA_GATHER_INSTALL, err=self.err, stream=stream)

    def run(self, stream, topk, q):
        """topk [B, 1, k] int32 (device); q: list of [B, 1, H, 576] bf16 per layer."""
        # the caller's tensors are read by work queued on other streams: keep the caching
        # allocator from reusing their memory before that work is done
        for t in [topk] + list(q):
            t.record_stream(stream)
            if self.aux:
                t.record_stream(self.aux_stream)
        po = self.plan_out[self.step_no % 2]
        if self.aux:
            stream.wait_event(self.plan_free[self.step_no % 2])
        self.plan(stream, topk, po)
        for l in range(self.layers):
            if self.aux:
                stream.wait_event(self.installed[l])
            self.serve(stream, topk, po, l)
            if self.aux:
                served = torch.cuda.Event()
                served.record(stream)
                self.aux_stream.wait_event(served)
                self.install(self.aux_stream, topk, po, l)
                self.installed[l].record(self.aux_stream)
            self.attend(stream, q[l], l)
            if not self.aux:
                self.install(stream, topk, po, l)
        if self.aux:
            self.plan_free[self.step_no % 2].record(self.aux_stream)
        self.step_no += 1

    def drain(self, stream):
        """Make `stream` wait for the installs still pending on the auxiliary stream."""
        if self.aux and self.step_no:
            stream.wait_event(self.plan_free[(self.step_no - 1) % 2])


class MtpDraftSteps:
    """MTP draft steps over one frozen selection (the first step's top-k): one plan, one
    serve of the selected rows (hits from the device pool, misses from the host rows), an
    attention per draft step with that step's queries, and the installs after the last
    draft step (the frozen selection needs nothing new from the pool meanwhile).  With
    `reuse`, every draft step reads the first serve's selection buffer; without it, each
    draft step serves the same rows again (history rows are immutable and the pool rows are
    unchanged until the installs, so both give the same bytes)."""

    def __init__(self, pg: PoolGroupStep, reuse: bool):
        self.pg, self.reuse = pg, reuse

    def run(self, stream, topk, q_steps):
        """topk [B, 1, k]; q_steps: per draft step, a list of per-layer queries.  Returns
        the per-step list of per-layer (o, lse) copies."""
        pg = self.pg
        po = pg.plan_out[0]
        outs = []
        for t in [topk] + [x for q in q_steps for x in q]:
            t.record_stream(stream)
        with torch.cuda.stream(stream):
            pg.plan(stream, topk, po)
            for d, q in enumerate(q_steps):
                for l in range(pg.layers):
                    if d == 0 or not self.reuse:
                        pg.serve(stream, topk, po, l)
                    pg.attend(stream, q[l], l)
                outs.append([(o.clone(), lse.clone()) for o, lse in zip(pg.o, pg.lse)])
            for l in range(pg.layers):
                pg.install(stream, topk, po, l)
        return outs


class MtpVerifyPoolStep:
    """One verify step of Sq query tokens (the main token and its drafts) over the device pool
    of a shared group.  With `union` (the de-duplicated multi-query gather): the union of the
    query tokens' selections is planned once for the group, and per layer its rows are served
    once, so a position several tokens select crosses the host link at most once; every token
    then attends over its own entries of the served union through its union indices.  Without
    `union`, every (token, entry) is served on its own, as dsa_gather_kv does for [B, Sq, k]
    selections.  Either way the plan is committed at plan time and the installs follow each
    layer's attention.

    host : list (one per layer) of Rows over the request-major host rows [B*L, 576]
    """

    def __init__(self, B, Sq, k, H, n_sets, ways, id_range, host, scale, union=True, device="cuda"):
        self.B, self.Sq, self.k, self.H, self.S, self.W = B, Sq, k, H, n_sets, ways
        self.host, self.scale, self.union = host, scale, union
        self.layers = len(host)
        dev = device
        cap = Sq * k
        self.cap = cap
        self.pool = [torch.zeros((B, n_sets * ways, 576), dtype=torch.bfloat16, device=dev) for _ in host]
        self.pids = torch.full((B, n_sets * ways), -1, dtype=torch.int32, device=dev)
        self.its = torch.full((B, id_range), -1, dtype=torch.int32, device=dev)
        self.ptr = torch.zeros((B, n_sets), dtype=torch.int32, device=dev)
        shape = (B, 1, cap) if union else (B, Sq, k)
        self.plan_out = dict(is_hit=torch.empty(shape, dtype=torch.uint8, device=dev),
                             slot=torch.empty(shape, dtype=torch.int32, device=dev),
                             mp=torch.empty((B, cap), dtype=torch.int32, device=dev),
                             ms=torch.empty((B, cap), dtype=torch.int32, device=dev),
                             mc=torch.empty(B, dtype=torch.int32, device=dev))
        self.uni = torch.empty((B, 1, cap), dtype=torch.int32, device=dev)
        self.count = torch.empty(B, dtype=torch.int32, device=dev)
        self.uidx = torch.empty((B, Sq, k), dtype=torch.int32, device=dev)
        self.sel = [torch.empty((B, cap, 576), dtype=torch.bfloat16, device=dev) for _ in host]
        self.sel_rows = [dsa.Rows(s, 1152, req_stride=cap) for s in self.sel]
        self.o = [torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device=dev) for _ in host]
        self.lse = [torch.empty((B, Sq, H), dtype=torch.float32, device=dev) for _ in host]
        self.ws = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(B, Sq, H, k)), dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(self, stream, topk, q):
        """topk [B, Sq, k] int32 (device, rows ascending); q: per layer [B, Sq, H, 576] bf16."""
        for t in [topk] + list(q):
            t.record_stream(stream)
        po = self.plan_out
        # the served entries: the union (one row) or every (token, entry)
        served = self.uni if self.union else topk
        if self.union:
            dsa.dsa_topk_union(topk, self.uni.view(self.B, self.cap), self.count, self.uidx, err=self.err,
                               stream=stream)
        dsa.dsa_plan(served, self.pids, self.its, self.ptr, self.S, self.W, po["is_hit"], po["slot"], po["mp"],
                     po["ms"], po["mc"], commit=True, err=self.err, stream=stream)
        for l in range(self.layers):
            sel4 = self.sel[l].view(served.shape + (576,))
            dsa.dsa_gather_kv(served, po["is_hit"], po["slot"], self.host[l], self.pool[l], sel4,
                              dsa.DSA_GATHER_SERVE, err=self.err, stream=stream,
                              sel_idx=None if self.union else self.uidx)
            # union: token t's entry j is union row uidx[t, j]; per entry: served row t * k + j
            dsa.dsa_sparse_mla_decode(q[l], self.uidx, self.sel_rows[l], self.scale, self.o[l], self.lse[l],
                                      ws=self.ws, err=self.err, stream=stream)
            dsa.dsa_gather_kv(served, po["is_hit"], po["slot"], None, self.pool[l], sel4,
                              dsa.DSA_GATHER_INSTALL, err=self.err, stream=stream)
