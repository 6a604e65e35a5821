"""Synthetic paged-decode workloads: shapes, structure and seeded draws.

Five workloads, named for what they are:

``tiny_fp32``            4 sequences, lengths {40, 17, 64, 1}, fp32, 8 query /
                         2 KV heads (GQA group 4), head dim 64, pool of 32 blocks.
``llama3_8b_b64``        Llama-3-8B attention shape (32 query / 8 KV heads, head
                         dim 128), bf16, batch 64, lengths uniform in
                         [512, 4096], pool sized exactly to the blocks in use.
``shared_prefix_b128``   bf16, batch 128, 64 query / 8 KV heads, head dim 128;
                         every table starts with the same 64 blocks (a
                         1024-token prefix), then unique suffix blocks for
                         suffix lengths uniform in [64, 2048]; sequence 1 is a
                         fork of sequence 0 (shares all its blocks, whose last
                         block is partly filled), so the next append hits a
                         shared partial block and needs a copy.
``quant_kv_32k_b16``     batch 16, 32 query / 8 KV heads, head dim 128, 32768
                         tokens each, bf16 source values with 1% of the
                         (KV head, channel) pairs of K scaled by 8, stored as
                         INT8 (``kv_dtype="i8"``), FP8-E4M3 (``"fp8e4m3"``),
                         FP8-E5M2 (``"fp8e5m2"``) or packed INT4 (``"i4"``)
                         codes with one scale per (block, KV head); bf16
                         queries.
``ctx128k_b4``           batch 4, Llama-3.1-70B attention shape (64 query / 8 KV
                         heads, head dim 128), bf16, 131072 tokens each,
                         512-token split-K partitions; ``streaming=True`` keeps
                         4 sink tokens plus the latest 4092.

Every workload can be shrunk with overrides (``S``, ``len_lo``/``len_hi``,
``fixed_len``, ...) for parity runs the CPU oracle finishes in seconds.
"""

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 4660


@dataclass
class Workload:
    name: str
    q_dtype: str            # "f32" | "bf16" | "f16"
    kv_dtype: str           # storage of the cache read by attention
    src_dtype: str          # dtype of the prompt K/V written by the slot write
    S: int
    Hq: int
    Hkv: int
    D: int
    BS: int = 16
    seed: int = SEED_BASE
    fixed_lens: tuple = ()          # explicit lengths, else uniform draw
    len_lo: int = 0
    len_hi: int = 0
    fixed_len: int = 0              # every sequence this long (when > 0)
    prefix_tokens: int = 0          # shared prefix length (multiple of BS)
    fork: tuple = ()                # (parent, child): child shares all parent blocks
    outlier_frac: float = 0.0       # fraction of K (head, channel) pairs scaled
    outlier_mult: float = 1.0
    pool_blocks: int = 0            # > 0: fixed pool size; 0: exactly what is used
    append: bool = True             # the decode step appends one token per sequence
    sink: int = 0
    window: int = 0
    partition_size: int = 0         # 0: library's choice
    # filled by instantiate()
    seq_lens: np.ndarray = field(default=None, repr=False)
    num_blocks: int = 0
    initial_order: np.ndarray = field(default=None, repr=False)
    outlier_pairs: np.ndarray = field(default=None, repr=False)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def sm_scale(self):
        return float(np.float32(1.0) / np.float32(math.sqrt(self.D)))


def _base(name):
    if name == "tiny_fp32":
        return Workload(name, "f32", "f32", "f32", S=4, Hq=8, Hkv=2, D=64,
                        seed=SEED_BASE + 0, fixed_lens=(40, 17, 64, 1), pool_blocks=32)
    if name == "llama3_8b_b64":
        return Workload(name, "bf16", "bf16", "bf16", S=64, Hq=32, Hkv=8, D=128,
                        seed=SEED_BASE + 1, len_lo=512, len_hi=4096)
    if name == "shared_prefix_b128":
        return Workload(name, "bf16", "bf16", "bf16", S=128, Hq=64, Hkv=8, D=128,
                        seed=SEED_BASE + 2, len_lo=64, len_hi=2048, prefix_tokens=1024,
                        fork=(0, 1))
    if name == "quant_kv_32k_b16":
        return Workload(name, "bf16", "i8", "bf16", S=16, Hq=32, Hkv=8, D=128,
                        seed=SEED_BASE + 3, fixed_len=32768, outlier_frac=0.01,
                        outlier_mult=8.0, append=False)
    if name == "ctx128k_b4":
        return Workload(name, "bf16", "bf16", "bf16", S=4, Hq=64, Hkv=8, D=128,
                        seed=SEED_BASE + 4, fixed_len=131072, partition_size=512)
    raise KeyError(name)


WORKLOADS = ("tiny_fp32", "llama3_8b_b64", "shared_prefix_b128", "quant_kv_32k_b16", "ctx128k_b4")


def _ceil_div(a, b):
    return -(-a // b)


def get_workload(name, streaming=False, **overrides):
    """The named workload with integer structure drawn (lengths, pool order,
    outlier channels).  ``overrides`` replace dataclass fields before the draw;
    ``streaming=True`` sets the 4-sink + 4092-window keep-mask."""
    w = _base(name)
    if streaming:
        overrides.setdefault("sink", 4)
        overrides.setdefault("window", 4092)
        # the partition size of a workload is for full attention; the
        # windowed variant reads ~3% of it and uses the library's choice
        overrides.setdefault("partition_size", 0)
    if overrides:
        w = dataclasses.replace(w, **overrides)
    rng = np.random.default_rng(w.seed)

    # -- lengths -----------------------------------------------------------
    if w.fixed_lens:
        lens = np.asarray(w.fixed_lens[: w.S], dtype=np.int64)
    elif w.fixed_len:
        lens = np.full(w.S, w.fixed_len, dtype=np.int64)
    else:
        lens = rng.integers(w.len_lo, w.len_hi + 1, size=w.S).astype(np.int64)
    if w.prefix_tokens:
        lens = lens + w.prefix_tokens              # drawn values are suffix lengths
    if w.fork:
        parent, child = w.fork
        if lens[parent] % w.BS == 0:               # parent's last block must be partial
            lens[parent] -= 1
        lens[child] = lens[parent]
    w.seq_lens = lens.astype(np.int32)

    # -- pool size and free-list order -------------------------------------
    extra = 1 if w.append else 0
    if w.pool_blocks:
        nb = w.pool_blocks
    else:
        # every sequence owns its blocks after the append, except that the
        # prefix blocks are counted once (in sequence 0) and a fork owns none
        pref = w.prefix_tokens // w.BS
        child = w.fork[1] if w.fork else -1
        nb = 0
        for s in range(w.S):
            if s == child:
                continue
            n = _ceil_div(int(lens[s]) + extra, w.BS)
            nb += n if (s == 0 or not pref) else n - pref
        if w.fork and w.append:
            nb += 1                                 # the copy-on-write block
    w.num_blocks = int(nb)
    w.initial_order = rng.permutation(w.num_blocks).astype(np.int32)

    # -- outlier channels of K --------------------------------------------
    n_out = int(round(w.outlier_frac * w.Hkv * w.D))
    w.outlier_pairs = np.sort(rng.choice(w.Hkv * w.D, size=n_out, replace=False)).astype(np.int64) \
        if n_out else np.zeros(0, dtype=np.int64)
    return w


def plan_ops(w):
    """How the block tables are built, as pool operations:

    ``("new", s, L)``        allocate fresh blocks for sequence s's L tokens;
    ``("share", s, p, n)``   sequence s starts with sequence p's first n blocks;
    ``("grow", s, L)``       allocate fresh blocks until s covers L tokens.

    Executed in order by each side's own pool.
    """
    ops = []
    pref = w.prefix_tokens // w.BS
    child = w.fork[1] if w.fork else -1
    for s in range(w.S):
        L = int(w.seq_lens[s])
        if s == child:
            parent = w.fork[0]
            ops.append(("share", s, parent, _ceil_div(int(w.seq_lens[parent]), w.BS)))
        elif pref and s != 0:
            ops.append(("share", s, 0, pref))
            ops.append(("grow", s, L))
        else:
            ops.append(("new", s, L))
    return ops


def prompt_tokens(w):
    """(seq_ids, positions) of every prompt token that gets written into the
    cache: all tokens of each sequence, except positions covered by shared
    blocks (the prefix is written once, by sequence 0; a fork writes none)."""
    seq_ids, pos = [], []
    child = w.fork[1] if w.fork else -1
    for s in range(w.S):
        if s == child:
            continue
        start = w.prefix_tokens if (w.prefix_tokens and s != 0) else 0
        L = int(w.seq_lens[s])
        seq_ids.append(np.full(L - start, s, dtype=np.int32))
        pos.append(np.arange(start, L, dtype=np.int32))
    return np.concatenate(seq_ids), np.concatenate(pos)


_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def draw_tensors(w, device="cpu"):
    """Seeded floating-point inputs for workload ``w`` on ``device``.

    Returns a dict of torch tensors:
      ``seq_ids``, ``positions`` int32 [T]   prompt tokens to write,
      ``key``, ``value``   [T, Hkv, D] in ``w.src_dtype``  their K / V,
      ``query``            [S, Hq, D]  in ``w.q_dtype``,
      ``new_key``, ``new_value`` [S, Hkv, D]  the decode step's new token.
    Values are N(0, 1) drawn in fp32 then rounded (RNE) to the storage type;
    K outlier (head, channel) pairs are multiplied in fp32 before rounding.
    """
    seq_ids, positions = prompt_tokens(w)
    T = int(seq_ids.size)
    g = torch.Generator(device=device)
    g.manual_seed(int(w.seed))
    sdt = _TORCH[w.src_dtype]

    def normal(shape, dt, outliers=False):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if outliers and w.outlier_pairs.size:
            flat = x.view(shape[0], -1)
            idx = torch.as_tensor(w.outlier_pairs, device=device)
            flat[:, idx] *= float(w.outlier_mult)
        return x.to(dt)

    # draw prompt K/V in chunks to bound the fp32 temporary
    key = torch.empty((T, w.Hkv, w.D), dtype=sdt, device=device)
    value = torch.empty((T, w.Hkv, w.D), dtype=sdt, device=device)
    chunk = max(1, (1 << 26) // (w.Hkv * w.D))
    for lo in range(0, T, chunk):
        n = min(chunk, T - lo)
        key[lo:lo + n] = normal((n, w.Hkv, w.D), sdt, outliers=True)
    for lo in range(0, T, chunk):
        n = min(chunk, T - lo)
        value[lo:lo + n] = normal((n, w.Hkv, w.D), sdt)
    query = normal((w.S, w.Hq, w.D), _TORCH[w.q_dtype])
    new_key = normal((w.S, w.Hkv, w.D), sdt, outliers=True)
    new_value = normal((w.S, w.Hkv, w.D), sdt)
    return {
        "seq_ids": torch.as_tensor(seq_ids, device=device),
        "positions": torch.as_tensor(positions, device=device),
        "key": key, "value": value, "query": query,
        "new_key": new_key, "new_value": new_value,
    }
