"""Hit rates of device-pool policies on the pool workload's synthetic top-k trajectory
(test infrastructure only; prints the table quoted in the design notes).

    python -m oracle.hit_rates

Average over requests and over steps 1..S-1 (step 0 starts from an empty pool) of
hits / k for: the previous step's set only, fully associative LRU pools of 8192 and 16384
ids, and set-associative FIFO pools of 8192 (1024 x 8, 512 x 16) and 16384 (1024 x 16)
entries.
"""
import numpy as np

import synth
from . import plan


def table():
    cfg = synth.spec(4)
    traj = synth.gen.topk_trajectory(cfg)             # [steps, B, k]
    S, B, k = traj.shape
    rows = {
        "previous step's set (k entries)": lambda t: plan.previous_set_hits(t),
        "LRU, 8192 entries": lambda t: plan.lru_hits(t, 8192),
        "LRU, 16384 entries": lambda t: plan.lru_hits(t, 16384),
        "FIFO 1024 sets x 8 ways (8192)": lambda t: plan.fifo_hits(t, 1024, 8, cfg.id_range),
        "FIFO 512 sets x 16 ways (8192)": lambda t: plan.fifo_hits(t, 512, 16, cfg.id_range),
        "FIFO 1024 sets x 16 ways (16384)": lambda t: plan.fifo_hits(t, 1024, 16, cfg.id_range),
    }
    out = {}
    for name, fn in rows.items():
        h = np.stack([fn(traj[:, b]) for b in range(B)])   # [B, S]
        out[name] = float(h[:, 1:].mean() / k)
    return out


if __name__ == "__main__":
    for name, rate in table().items():
        print(f"{name:36s} {100 * rate:6.2f}%")
