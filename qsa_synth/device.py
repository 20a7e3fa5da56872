"""Device-resident synthetic inputs of a workload (torch tensors on the GPU).

Small tensors are generated on the host and uploaded; index keys and KV
pools are filled on the GPU by the generator's fill kernels (bit-identical to
the host generator). The KV pools of an offload workload live in pinned host
memory and are filled through a device staging buffer.
"""
from __future__ import annotations

import numpy as np
import torch

from . import GEOM, HostInputs, Workload, host_inputs
from . import fill


class DeviceInputs:
    def __init__(self, wl: Workload, device="cuda:0", kv_host=None, layers=None, hi: HostInputs = None):
        self.wl = wl
        self.hi = hi if hi is not None else host_inputs(wl)
        self.device = torch.device(device)
        self.kv_host = wl.kv_host if kv_host is None else kv_host
        self.n_layers = wl.layers if layers is None else layers
        hi, dev, g = self.hi, self.device, GEOM
        lay = hi.lay
        self.batch = wl.batch
        self.max_ctx = int(lay.ctx.max())
        self.ctx = torch.from_numpy(lay.ctx.astype(np.int32)).to(dev)
        self.row0 = torch.from_numpy(lay.row0.astype(np.int64)).to(dev)
        self.pt = torch.from_numpy(np.ascontiguousarray(lay.pt)).to(dev)
        self.pt_stride = int(lay.pt.shape[1])
        self.n_slots = int(lay.n_slots)
        self.n_rows = int(lay.n_rows)
        L = self.n_layers
        self.q_idx = torch.from_numpy(hi.q_idx[:L].view(np.int16)).to(dev)     # [L][B][4][64] bf16 bits
        self.w_idx = torch.from_numpy(hi.w[:L]).to(dev)                        # [L][B][4]
        self.q = torch.from_numpy(hi.q[:L].view(np.int16)).to(dev)             # [L][B][16][256]
        self.keys = torch.empty((L, self.n_rows, g.idx_dim), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((L, self.n_rows), dtype=torch.int16, device=dev)
        for l in range(L):
            fill.fill_index_layer(hi, l, self.keys[l], self.scales[l])
        if self.kv_host:
            self.pool = torch.empty((L, self.n_slots, g.row_elems), dtype=torch.int16, pin_memory=True)
            chunk = 1 << 18
            tmp = torch.empty((chunk, g.row_elems), dtype=torch.int16, device=dev)
            for l in range(L):
                for a in range(0, self.n_slots, chunk):
                    n = min(chunk, self.n_slots - a)
                    fill.fill_kv_rows(tmp, a, n, l, wl.seed)
                    self.pool[l, a:a + n].copy_(tmp[:n])
            del tmp
        else:
            self.pool = torch.empty((L, self.n_slots, g.row_elems), dtype=torch.int16, device=dev)
            for l in range(L):
                fill.fill_kv_rows(self.pool[l], 0, self.n_slots, l, wl.seed)
        self.out = torch.zeros((L, self.batch, g.n_q_heads, g.head_dim), dtype=torch.float32, device=dev)
        torch.cuda.synchronize(dev)

    # algorithmic bytes of one decode step given the per-(layer, seq) token counts
    def index_bytes_per_layer(self) -> int:
        return int(self.hi.lay.ctx.sum()) * GEOM.index_row_bytes
