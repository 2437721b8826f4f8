"""Test helpers: the device uploads of synth.device and the package's step orchestration,
plus conversions the checks use.  Only plumbing lives here; the numerical checks are in the
test files, against the oracle."""
import numpy as np
import torch

from paged_kv_cache_indexer_amd.pipeline import (  # noqa: F401
    DecodeStep, HipMark, LayerCaches, MtpDraftSteps, PoolGroupStep, host_device_ptr)
from synth.device import DEV, DevWorkload, t_f32, t_i32, t_u8, t_u16_as_bf16  # noqa: F401


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)

