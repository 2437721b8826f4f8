"""Device copies of a seeded workload: uploads its byte arrays into torch tensors on the GPU
and describes the paged caches as libdsa row stores.  Plumbing only (no arithmetic of the
method); the benchmark and the GPU tests share it.
"""
import numpy as np
import torch

import paged_kv_cache_indexer_amd as dsa
from paged_kv_cache_indexer_amd.pipeline import DecodeStep, LayerCaches

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
        self.q_dtype = {"f32": dsa.DSA_F32, "bf16": dsa.DSA_BF16, "e4m3": dsa.DSA_E4M3}[wl.idx_q_dtype]
        if wl.idx_q_dtype == "f32":
            self.idx_q = t_f32(wl.idx_q)
        elif wl.idx_q_dtype == "bf16":
            self.idx_q = t_u16_as_bf16(wl.idx_q)
        else:
            self.idx_q = t_u8(wl.idx_q)
        D = wl.idx_k.shape[-1]
        if wl.idx_k_dtype == "f32":
            self.idx_k, self.k_dtype, row_bytes = t_f32(wl.idx_k), dsa.DSA_F32, D * 4
            self.k_scale = t_f32(wl.idx_k_scale) if wl.idx_k_scale is not None else None
        elif wl.idx_k_dtype == "mxfp4":                # packed E2M1 rows + E8M0 block scales
            self.idx_k, self.k_dtype, row_bytes = t_u8(wl.idx_k), dsa.DSA_MXFP4, D
            self.k_scale = t_u8(wl.idx_k_scale)
        else:
            self.idx_k, self.k_dtype, row_bytes = t_u8(wl.idx_k), dsa.DSA_E4M3, D
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

    def layer_caches(self, layers: int = 1):
        """`layers` distinct device copies of the per-layer caches (indexer keys, their scales,
        latent rows); the first is this workload's own."""
        out = [LayerCaches(self.keys, self.k_scale, self.rows)]
        for _ in range(layers - 1):
            k = self.idx_k.clone()
            ks = self.k_scale.clone() if self.k_scale is not None else None
            kv = self.kv.clone()
            out.append(LayerCaches(dsa.Rows(k, self.keys.c.row_bytes, self.page_table, self.wl.page_size), ks,
                                   dsa.Rows(kv, 1152, self.page_table, self.wl.page_size)))
        return out

    def decode_step(self, layers: int = 1, o_dtype=torch.bfloat16, fused: bool = True) -> DecodeStep:
        """A DecodeStep over this workload, rotating through `layers` copies of its caches."""
        return DecodeStep(self.idx_q, self.idx_w, self.seq_lens, self.mla_q, self.layer_caches(layers),
                          self.wl.topk, self.wl.scale, self.Lmax, self.k_dtype, self.q_dtype, err=self.err,
                          o_dtype=o_dtype, fused=fused)
