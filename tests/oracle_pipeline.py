"""Runs a whole decode step of a workload through the CPU oracle.

Test helper: uses only ``oracle`` and ``workloads``.  Steps, in the order a
serving engine takes them:

1. build block tables from the workload's pool plan with the oracle pool;
2. write every prompt token into a poisoned cache with the oracle slot write;
3. (quantised workloads) quantise every used block per (block, KV head);
4. decode step: append one slot per sequence (copy-on-write if shared), copy
   blocks, write the new token, then attend over length + 1.
"""

import numpy as np
import torch

import oracle
from oracle import attention, paging, quant
from plan import build_tables

POISON = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "f16": np.uint16(0x7E00),
          "i8": np.int8(-128), "fp8e4m3": np.uint8(0x7F), "fp8e5m2": np.uint8(0x7F), "i4": np.uint8(0x88)}
RAW_NP = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "i8": np.int8, "fp8e4m3": np.uint8,
          "fp8e5m2": np.uint8, "i4": np.uint8}


def to_raw(t, dtype):
    """torch tensor -> numpy array of storage words for ``dtype``."""
    t = t.detach().cpu()
    if dtype in ("bf16", "f16"):
        return t.view(torch.int16).numpy().view(np.uint16)
    if dtype == "f32":
        return t.numpy().astype(np.float32)
    if dtype == "i8":
        return t.numpy().astype(np.int8)
    if dtype in ("fp8e4m3", "fp8e5m2", "i4"):
        return t.view(torch.uint8).numpy()
    raise ValueError(dtype)


def pad_tables(tables, width, fill=0):
    out = np.full((len(tables), width), fill, dtype=np.int32)
    for s, t in enumerate(tables):
        out[s, : len(t)] = t
    return out


class OracleRun:
    """State of the oracle after prefill and after the decode step."""

    def __init__(self, w, tensors, seqs=None, do_step=True):
        self.w = w
        self.pool = oracle.pool.BlockPool(w.num_blocks, w.initial_order)
        self.tables = build_tables(w, self.pool)
        shape = (w.num_blocks, w.BS, w.Hkv, w.D)
        src = w.src_dtype
        self.k_cache = np.full(shape, POISON[src], dtype=RAW_NP[src])
        self.v_cache = np.full(shape, POISON[src], dtype=RAW_NP[src])
        bt = pad_tables(self.tables, max(len(t) for t in self.tables) + 1)
        seq_ids = tensors["seq_ids"].cpu().numpy()
        pos = tensors["positions"].cpu().numpy()
        self.prompt_slots = paging.slot_mapping(bt, seq_ids, pos, w.BS)
        paging.reshape_and_cache(self.k_cache, to_raw(tensors["key"], src), self.prompt_slots, w.BS)
        paging.reshape_and_cache(self.v_cache, to_raw(tensors["value"], src), self.prompt_slots, w.BS)
        self.k_scales = self.v_scales = None
        self.lens = w.seq_lens.astype(np.int64).copy()
        if w.kv_dtype in quant.CODE_DTYPES:
            used = sorted({b for t in self.tables for b in t})
            kv = oracle.codecs.decode(self.k_cache, src)
            vv = oracle.codecs.decode(self.v_cache, src)
            self.k_src, self.v_src = self.k_cache, self.v_cache
            self.k_cache, self.k_scales = quant.quantize_cache_blocks(kv, w.kv_dtype, used)
            self.v_cache, self.v_scales = quant.quantize_cache_blocks(vv, w.kv_dtype, used)
            unused = np.setdiff1d(np.arange(w.num_blocks), used)
            for arr in (self.k_cache, self.v_cache):
                arr[unused] = POISON[w.kv_dtype]
        self.step_slots = None
        self.cow = []
        if do_step and w.append:
            self.decode_step(tensors)

    def decode_step(self, tensors):
        w = self.w
        slots = np.empty(w.S, dtype=np.int64)
        for s in range(w.S):
            slot, cow = self.pool.append(self.tables[s], int(self.lens[s]), w.BS)
            slots[s] = slot
            if cow is not None:
                self.cow.append(cow)
        arrays = [self.k_cache, self.v_cache]
        if self.k_scales is not None:
            arrays += [self.k_scales, self.v_scales]
        self.cow_src_before = [(self.k_cache[src].copy(), self.v_cache[src].copy()) for src, _ in self.cow]
        paging.copy_blocks(arrays, self.cow)
        paging.reshape_and_cache(self.k_cache, to_raw(tensors["new_key"], w.src_dtype), slots, w.BS)
        paging.reshape_and_cache(self.v_cache, to_raw(tensors["new_value"], w.src_dtype), slots, w.BS)
        self.step_slots = slots
        self.lens = self.lens + 1

    def block_tables(self, width=None):
        width = width or max(len(t) for t in self.tables)
        return pad_tables(self.tables, width)

    def decode(self, query_raw, seqs=None, partition_size=None):
        w = self.w
        return attention.paged_decode(
            query_raw, w.q_dtype, self.k_cache, self.v_cache, w.kv_dtype,
            self.block_tables(), self.lens, w.BS, w.sm_scale,
            self.k_scales, self.v_scales, w.sink, w.window, seqs=seqs)
