"""Device staging of synthetic cases for the HIP library (tests, bench, smoke).

Copies a case's rows into a paged pool on the GPU, builds the descriptor and
plan, allocates outputs and workspace, and calls the library through its
binding.  Layout work only; no attention arithmetic.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

import invariant_split_kv_amd as isk

from . import synth


def _u16_to_bf16(arr: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def make_desc(case, split_mode=isk.SPLIT_PER_ROW, out_f32=False, check_inputs=False,
              split_tokens: Optional[int] = None) -> isk.IskDesc:
    pg = case.paging
    st = case.split_tokens if split_tokens is None else split_tokens
    if isinstance(case, synth.GqaCase):
        return isk.IskDesc(isk.KIND_GQA, case.hq, case.hkv, case.d, case.d, pg.page_size, pg.num_pages,
                           pg.max_pages_per_row, 0, split_mode, st, int(out_f32), int(check_inputs), case.scale)
    return isk.IskDesc(isk.KIND_MLA, case.hq, 1, synth.MLA_DQK, synth.MLA_DV, pg.page_size, pg.num_pages,
                       pg.max_pages_per_row, case.topk_width, split_mode, st, int(out_f32), int(check_inputs),
                       case.scale)


def device_pool(case, device="cuda", fill: Optional[int] = None) -> torch.Tensor:
    """The case's paged KV pool on the device.  Slots no row uses hold 0, or
    the bf16 bit pattern `fill` when given (to show such slots are never read)."""
    pg = case.paging
    if isinstance(case, synth.GqaCase):
        host = case.pool_bits()
        if fill is not None:
            used = np.zeros(pg.num_pages * pg.page_size, bool)
            for b, L in enumerate(case.lens):
                if L:
                    used[pg.token_slots(b, np.arange(int(L)))] = True
            tok_major = host.transpose(0, 3, 1, 2, 4).reshape(pg.num_pages * pg.page_size, -1)
            tok_major[~used] = fill
            host = np.ascontiguousarray(
                tok_major.reshape(pg.num_pages, pg.page_size, 2, case.hkv, case.d).transpose(0, 2, 3, 1, 4))
        return _u16_to_bf16(host, device)
    fill_i16 = 0 if fill is None else int(np.array(fill, dtype=np.uint16).view(np.int16))
    flat = torch.full((pg.num_pages * pg.page_size, synth.MLA_DQK), fill_i16, dtype=torch.int16, device=device)
    for b, r in enumerate(case.rows):
        if case.sparse:
            j = case.placed_slots(b)
            if len(j) == 0:
                continue
            slots, vals = pg.token_slots(b, r.topk_idx[j]), r.gathered[j]
        else:
            L = int(case.lens[b])
            if L == 0:
                continue
            slots, vals = pg.token_slots(b, np.arange(L)), r.latent
        flat[torch.from_numpy(slots).to(device)] = torch.from_numpy(np.ascontiguousarray(vals).view(np.int16)).to(device)
    return flat.view(torch.bfloat16).view(pg.num_pages, pg.page_size, synth.MLA_DQK)


class DeviceCase:
    """A case staged on the GPU together with its plan and buffers."""

    def __init__(self, case, device="cuda", split_mode=isk.SPLIT_PER_ROW, out_f32=False, check_inputs=False,
                 split_tokens: Optional[int] = None, pool: Optional[torch.Tensor] = None,
                 fill: Optional[int] = None, bands=None):
        self.case = case
        self.device = device
        self.desc = make_desc(case, split_mode, out_f32, check_inputs, split_tokens)
        self.q = _u16_to_bf16(case.q_bits(), device)
        self.pool = device_pool(case, device, fill) if pool is None else pool
        self.block_table = torch.from_numpy(case.paging.block_table).to(device)
        self.lens_host = np.asarray(case.lens, dtype=np.int32)
        self.lens = torch.from_numpy(self.lens_host).to(device)
        sparse = isinstance(case, synth.MlaCase) and case.sparse
        self.topk_len_host = case.topk_len() if sparse else None
        self.topk_idx = torch.from_numpy(case.topk_idx()).to(device) if sparse else None
        self.topk_len = torch.from_numpy(self.topk_len_host).to(device) if sparse else None
        self.extra = getattr(case, "extra", None)
        if self.extra is not None:
            x = self.extra
            self.x_pool = device_pool(x, device, fill)
            self.x_block_table = torch.from_numpy(x.paging.block_table).to(device)
            self.x_lens = torch.from_numpy(np.asarray(x.lens, dtype=np.int32)).to(device)
            self.x_topk_idx = torch.from_numpy(x.topk_idx()).to(device)
            self.x_topk_len_host = x.topk_len()
            self.x_topk_len = torch.from_numpy(self.x_topk_len_host).to(device)
            xdesc = isk.IskExtraDesc(x.paging.page_size, x.paging.num_pages, x.paging.max_pages_per_row,
                                     x.topk_width)
            self.plan = isk.Plan(self.desc, self.lens_host, self.topk_len_host, extra=xdesc,
                                 extra_topk_len_host=self.x_topk_len_host)
        else:
            self.plan = isk.Plan(self.desc, self.lens_host, self.topk_len_host, bands=bands)
        dv = self.desc.head_dim_v
        self.out = torch.empty((case.batch, case.hq, dv), dtype=torch.float32 if out_f32 else torch.bfloat16,
                               device=device)
        self.lse = torch.empty((case.batch, case.hq), dtype=torch.float32, device=device)
        self.ws_bytes = max(self.plan.workspace_bytes, 256)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    def run(self, stream=None) -> None:
        if self.extra is not None:
            isk.attn_decode_extra(self.plan.handle, self.q, self.pool, self.block_table, self.lens, self.topk_idx,
                                  self.topk_len, self.x_pool, self.x_block_table, self.x_lens, self.x_topk_idx,
                                  self.x_topk_len, self.out, self.lse, self.workspace, self.ws_bytes, stream)
            return
        isk.attn_decode(self.plan.handle, self.q, self.pool, self.block_table, self.lens, self.topk_idx,
                        self.topk_len, self.out, self.lse, self.workspace, self.ws_bytes, stream)

    def result(self):
        """(out as float64 numpy, lse as float64 numpy, raw out bits, raw lse bits)."""
        torch.cuda.synchronize()
        out = self.out.float().cpu().numpy().astype(np.float64)
        lse = self.lse.cpu().numpy().astype(np.float64)
        bits = self.out.view(torch.int16 if self.out.dtype == torch.bfloat16 else torch.int32).cpu().numpy().copy()
        lbits = self.lse.view(torch.int32).cpu().numpy().copy()
        return out, lse, bits, lbits

    def close(self) -> None:
        self.plan.close()


def kv_bytes(case) -> int:
    """Algorithmic KV bytes of one call: each attended token's K and V (GQA,
    per kv head) or its latent row (MLA) read once."""
    if isinstance(case, synth.GqaCase):
        return int(np.sum(case.lens)) * case.hkv * case.d * 2 * 2
    if case.sparse:
        n = int(np.sum(case.topk_len()))
        if getattr(case, "extra", None) is not None:
            n += int(np.sum(case.extra.topk_len()))
        return n * synth.MLA_DQK * 2
    return int(np.sum(case.lens)) * synth.MLA_DQK * 2


def io_bytes(case) -> int:
    """q read, out and lse written (bf16 out), block table and index reads."""
    if isinstance(case, synth.GqaCase):
        d_qk = d_v = case.d
    else:
        d_qk, d_v = synth.MLA_DQK, synth.MLA_DV
    b = case.batch * case.hq * (d_qk * 2 + d_v * 2 + 4)
    pages = sum(math.ceil(int(L) / case.paging.page_size) for L in case.lens)
    b += pages * 4 + case.batch * 4
    if isinstance(case, synth.MlaCase) and case.sparse:
        b += int(np.sum(case.topk_len())) * 4 + case.batch * 4
    if getattr(case, "extra", None) is not None:
        x = case.extra
        b += sum(math.ceil(int(L) / x.paging.page_size) for L in x.lens) * 4 + x.batch * 4
        b += int(np.sum(x.topk_len())) * 4 + x.batch * 4
    return b
