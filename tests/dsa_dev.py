"""Test helpers: upload a seeded workload to the GPU and run libdsa stages on it.

Only plumbing lives here (tensor uploads and calls through the C ABI binding); the
numerical checks are in the test files, against the oracle.
"""
import numpy as np
import torch

import paged_kv_cache_indexer_amd as dsa

DEV = "cuda"


def t_u16_as_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def t_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def t_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def t_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


class DevWorkload:
    """Device copies of a synth.Workload's indexer and MLA inputs."""

    def __init__(self, wl, with_kv: bool = True):
        self.wl = wl
        self.B, self.Sq = wl.B, wl.Sq
        self.seq_lens = t_i32(wl.seq_lens)
        self.page_table = t_i32(np.where(wl.page_table >= 0, wl.page_table, 0)) if wl.page_table.size else None
        self.Lmax = int(wl.seq_lens.max())
        if wl.idx_q_dtype == "f32":
            self.idx_q, self.k_dtype = t_f32(wl.idx_q), dsa.DSA_F32
            self.idx_k = t_f32(wl.idx_k)
            row_bytes = wl.idx_k.shape[-1] * 4
        else:
            self.idx_q = t_u16_as_bf16(wl.idx_q) if wl.idx_q_dtype == "bf16" else t_u8(wl.idx_q)
            self.k_dtype = dsa.DSA_E4M3
            self.idx_k = t_u8(wl.idx_k)
            row_bytes = wl.idx_k.shape[-1]
        if wl.idx_k_dtype == "f32":
            self.idx_k = t_f32(wl.idx_k)
            self.k_dtype = dsa.DSA_F32
            row_bytes = wl.idx_k.shape[-1] * 4
        self.q_dtype = {"f32": dsa.DSA_F32, "bf16": dsa.DSA_BF16, "e4m3": dsa.DSA_E4M3}[wl.idx_q_dtype]
        if wl.idx_k_dtype == "mxfp4":                  # packed E2M1 rows + E8M0 block scales
            self.k_dtype = dsa.DSA_MXFP4
            self.k_scale = t_u8(wl.idx_k_scale)
        else:
            self.k_scale = t_f32(wl.idx_k_scale) if wl.idx_k_scale is not None else None
        self.idx_w = t_f32(wl.idx_w)
        self.keys = dsa.Rows(self.idx_k, row_bytes, self.page_table, wl.page_size)
        self.mla_q = t_u16_as_bf16(wl.mla_q)
        if with_kv and wl.kv is not None:
            self.kv = t_u16_as_bf16(wl.kv)
            self.rows = dsa.Rows(self.kv, 1152, self.page_table, wl.page_size)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)

    def scores(self, ready=None):
        sc = torch.full((self.B, self.Sq, self.Lmax), float("nan"), dtype=torch.float32, device=DEV)
        dsa.dsa_indexer_scores(self.idx_q, self.idx_w, self.keys, self.k_scale, self.seq_lens, sc,
                               k_dtype=self.k_dtype, err=self.err, ready=ready, q_dtype=self.q_dtype)
        return sc

    def topk(self, sc, k=None):
        k = k or self.wl.topk
        idx = torch.empty((self.B, self.Sq, k), dtype=torch.int32, device=DEV)
        dsa.dsa_topk(sc, self.seq_lens, idx)
        return idx

    def mla(self, idx, o_dtype=torch.bfloat16, rows=None):
        H = self.wl.mla_q.shape[2]
        k = idx.shape[-1]
        o = torch.empty((self.B, self.Sq, H, 512), dtype=o_dtype, device=DEV)
        lse = torch.empty((self.B, self.Sq, H), dtype=torch.float32, device=DEV)
        nbytes = dsa.dsa_sparse_mla_workspace_size(self.B, self.Sq, H, k)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
        dsa.dsa_sparse_mla_decode(self.mla_q, idx, rows or self.rows, self.wl.scale, o, lse, ws=ws, err=self.err)
        return o, lse


class HipMark:
    """A HIP timing event recorded on a stream; `external=True` records it as an external
    event node when the stream is being captured into a graph, so its time stays readable
    after each replay."""

    _hip = None

    def __init__(self, external: bool = False):
        import ctypes
        if HipMark._hip is None:
            HipMark._hip = ctypes.CDLL("libamdhip64.so")
            HipMark._hip.hipEventRecordWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
            HipMark._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                         ctypes.c_void_p]
        self.ev = ctypes.c_void_p()
        rc = HipMark._hip.hipEventCreate(ctypes.byref(self.ev))
        assert rc == 0, f"hipEventCreate failed ({rc})"
        self.flags = 1 if external else 0          # hipEventRecordExternal

    def record(self, stream):
        rc = HipMark._hip.hipEventRecordWithFlags(self.ev, stream.cuda_stream, self.flags)
        assert rc == 0, f"hipEventRecordWithFlags failed ({rc})"

    def elapsed_ms(self, end: "HipMark") -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = HipMark._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        assert rc == 0, f"hipEventElapsedTime failed ({rc})"
        return ms.value


def host_device_ptr(t: torch.Tensor) -> int:
    """Device alias of a pinned host tensor (hipHostGetDevicePointer)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    dptr = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
    assert rc == 0, f"hipHostGetDevicePointer failed ({rc})"
    return dptr.value


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class DecodeStep:
    """One decode step (indexer -> top-k -> sparse MLA) over fixed device buffers.

    All buffers are allocated once, so the step can be captured into a HIP graph and
    replayed.  `run(stream, marks)` enqueues the three entry points on `stream`; if
    `marks` (four objects with a `record(stream)` method, e.g. HipMark) is given, they are
    recorded before, between and after the stages.
    """

    def __init__(self, dw: DevWorkload, layers: int = 1):
        """layers > 1: that many distinct device copies of the per-layer caches (indexer keys,
        their scales, latent rows); `run(..., layer=i)` uses copy i % layers.  Successive
        layers of a model read different caches, so rotating keeps a step from finding the
        previous step's cache bytes in the last-level cache."""
        wl = dw.wl
        self.dw = dw
        self.caches = [(dw.keys, dw.k_scale, dw.rows)]
        for _ in range(layers - 1):
            k = dw.idx_k.clone()
            ks = dw.k_scale.clone() if dw.k_scale is not None else None
            kv = dw.kv.clone()
            keys = dsa.Rows(k, dw.keys.c.row_bytes, dw.page_table, wl.page_size)
            rows = dsa.Rows(kv, 1152, dw.page_table, wl.page_size)
            self.caches.append((keys, ks, rows))
        B, Sq, L, k = dw.B, dw.Sq, dw.Lmax, wl.topk
        H = wl.mla_q.shape[2]
        self.scores = torch.empty((B, Sq, L), dtype=torch.float32, device=DEV)
        self.idx = torch.empty((B, Sq, k), dtype=torch.int32, device=DEV)
        self.o = torch.empty((B, Sq, H, 512), dtype=torch.bfloat16, device=DEV)
        self.lse = torch.empty((B, Sq, H), dtype=torch.float32, device=DEV)
        self.ws_mla = torch.empty(max(1, dsa.dsa_sparse_mla_workspace_size(B, Sq, H, k)), dtype=torch.uint8,
                                  device=DEV)
        self.ws_topk = torch.empty(max(1, dsa.dsa_topk_workspace_size(B, Sq, k, L)), dtype=torch.uint8, device=DEV)

    def stage(self, name, stream, layer=0):
        """Enqueue one stage ("indexer", "topk" or "mla") of the step on `stream`."""
        dw = self.dw
        keys, k_scale, rows = self.caches[layer % len(self.caches)]
        if name == "indexer":
            dsa.dsa_indexer_scores(dw.idx_q, dw.idx_w, keys, k_scale, dw.seq_lens, self.scores,
                                   k_dtype=dw.k_dtype, err=dw.err, q_dtype=dw.q_dtype, stream=stream)
        elif name == "topk":
            dsa.dsa_topk(self.scores, dw.seq_lens, self.idx, ws=self.ws_topk, stream=stream)
        elif name == "mla":
            dsa.dsa_sparse_mla_decode(dw.mla_q, self.idx, rows, dw.wl.scale, self.o, self.lse, ws=self.ws_mla,
                                      err=dw.err, stream=stream)
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

    With `aux_install`, each layer's install runs on a second stream: it waits for that
    layer's serve (it reads the served rows) and overlaps the layer's attention, and the
    next step's serve of the layer waits for it (it reads pool rows the install writes and
    overwrites the served rows the install reads).  The plan outputs alternate between two
    buffers, so the next step's plan never overwrites what a pending install still reads.

    host  : list (one per layer) of Rows over the request-major host rows [B*L, 576]
    """

    def __init__(self, B, k, H, n_sets, ways, id_range, host, scale, aux_install=False):
        self.B, self.k, self.H, self.S, self.W, self.idr = B, k, H, n_sets, ways, id_range
        self.host, self.scale, self.aux = host, scale, aux_install
        self.layers = len(host)
        dev = DEV
        self.pool = [torch.zeros((B, n_sets * ways, 576), dtype=torch.bfloat16, device=dev) for _ in host]
        self.sel = [torch.empty((B, 1, k, 576), dtype=torch.bfloat16, device=dev) for _ in host]
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
        self.ident = torch.arange(k, dtype=torch.int32, device=dev).repeat(B, 1).view(B, 1, k)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.aux_stream = torch.cuda.Stream() if aux_install else None
        self.installed = [torch.cuda.Event() for _ in host]          # layer l's last install
        self.plan_free = [torch.cuda.Event() for _ in range(2)]      # installs of the buffer's last step
        self.step_no = 0

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
        with torch.cuda.stream(stream):
            dsa.dsa_plan(topk, self.pids, self.its, self.ptr, self.S, self.W, po["is_hit"], po["slot"], po["mp"],
                         po["ms"], po["mc"], commit=True, err=self.err, stream=stream)
        for l in range(self.layers):
            if self.aux:
                stream.wait_event(self.installed[l])
            dsa.dsa_gather_kv(topk, po["is_hit"], po["slot"], self.host[l], self.pool[l], self.sel[l],
                              dsa.DSA_GATHER_SERVE, err=self.err, stream=stream)
            if self.aux:
                served = torch.cuda.Event()
                served.record(stream)
                self.aux_stream.wait_event(served)
                dsa.dsa_gather_kv(topk, po["is_hit"], po["slot"], None, self.pool[l], self.sel[l],
                                  dsa.DSA_GATHER_INSTALL, err=self.err, stream=self.aux_stream)
                self.installed[l].record(self.aux_stream)
            dsa.dsa_sparse_mla_decode(q[l], self.ident, dsa.Rows(self.sel[l], 1152, req_stride=self.k), self.scale,
                                      self.o[l], self.lse[l], ws=self.ws, err=self.err, stream=stream)
            if not self.aux:
                dsa.dsa_gather_kv(topk, po["is_hit"], po["slot"], None, self.pool[l], self.sel[l],
                                  dsa.DSA_GATHER_INSTALL, err=self.err, stream=stream)
        if self.aux:
            self.plan_free[self.step_no % 2].record(self.aux_stream)
        self.step_no += 1


class MtpDraftSteps:
    """MTP draft steps over one frozen selection (the first step's top-k): one plan, one
    serve of the selected rows (hits from the device pool, misses from the host rows), an
    attention per draft step with that step's queries, and the installs after the last
    draft step (the frozen selection needs nothing new from the pool meanwhile).  With
    `reuse`, every draft step reads the first serve's selection buffer; without it, each
    draft step serves the same rows again (history rows are immutable and the pool rows are
    unchanged until the installs, so both give the same bytes)."""

    def __init__(self, pg: "PoolGroupStep", reuse: bool):
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
            dsa.dsa_plan(topk, pg.pids, pg.its, pg.ptr, pg.S, pg.W, po["is_hit"], po["slot"], po["mp"], po["ms"],
                         po["mc"], commit=True, err=pg.err, stream=stream)
            for d, q in enumerate(q_steps):
                for l in range(pg.layers):
                    if d == 0 or not self.reuse:
                        dsa.dsa_gather_kv(topk, po["is_hit"], po["slot"], pg.host[l], pg.pool[l], pg.sel[l],
                                          dsa.DSA_GATHER_SERVE, err=pg.err, stream=stream)
                    dsa.dsa_sparse_mla_decode(q[l], pg.ident, dsa.Rows(pg.sel[l], 1152, req_stride=pg.k), pg.scale,
                                              pg.o[l], pg.lse[l], ws=pg.ws, err=pg.err, stream=stream)
                outs.append([(o.clone(), lse.clone()) for o, lse in zip(pg.o, pg.lse)])
            for l in range(pg.layers):
                dsa.dsa_gather_kv(topk, po["is_hit"], po["slot"], None, pg.pool[l], pg.sel[l],
                                  dsa.DSA_GATHER_INSTALL, err=pg.err, stream=stream)
        return outs
