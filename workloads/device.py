"""Upload a workload to a GPU as torch tensors (data movement only).

The pools are allocated on the device, filled with the poison code and only
the referenced token rows are scattered in, so host memory stays at the size
of the real tokens even for the 256K-page pools.
"""

from dataclasses import dataclass

import numpy as np
import torch

from .quantize import POISON_CODE


@dataclass
class DeviceWorkload:
    q: torch.Tensor             # float16 [B, Hq, D]
    k_pages: torch.Tensor       # uint8 [num_pages, Hkv, P, D]
    v_pages: torch.Tensor
    block_table: torch.Tensor   # int32 [B, max_pages_per_seq]
    context_lens: torch.Tensor  # int32 [B]
    scale: float


def to_device(w, device="cuda") -> DeviceWorkload:
    dev = torch.device(device)
    shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
    k = torch.full(shape, POISON_CODE, dtype=torch.uint8, device=dev)
    v = torch.full(shape, POISON_CODE, dtype=torch.uint8, device=dev)
    for b in range(w.batch):
        n = int(w.context_lens[b])
        if n <= 0:
            continue
        pg, slot = w.token_locations(b)
        pg_t = torch.from_numpy(pg).to(dev)
        slot_t = torch.from_numpy(slot.astype(np.int64)).to(dev)
        k[pg_t, :, slot_t, :] = torch.from_numpy(w.k_tokens[b]).to(dev)
        v[pg_t, :, slot_t, :] = torch.from_numpy(w.v_tokens[b]).to(dev)
    return DeviceWorkload(
        q=torch.from_numpy(w.q).to(dev),
        k_pages=k, v_pages=v,
        block_table=torch.from_numpy(w.block_table).to(dev),
        context_lens=torch.from_numpy(w.context_lens).to(dev),
        scale=w.scale)
