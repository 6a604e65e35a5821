"""Pins the CPU oracle to what the pages print and to closed forms.

Every fixture under tests/golden/ names the page and section it comes from.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import attention, codecs, paging, pool, quant, sizes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# addressing (t13_4 block-table example)
# --------------------------------------------------------------------------

def test_block_table_example():
    g = golden("block_table_example.json")
    bs, L, table = g["block_size"], g["seq_len"], g["block_table"]
    assert paging.blocks_needed(L, bs) == g["num_blocks_used"]
    assert L - (g["num_blocks_used"] - 1) * bs == g["tokens_in_last_block"]
    for logical, (t0, t1) in enumerate(g["logical_token_ranges"]):
        for t in range(t0, t1 + 1):
            slot = paging.slot_of(table, t, bs)
            assert slot // bs == table[logical]
            assert slot % bs == t - t0
    # slots of the whole sequence: 112..127, 32..47, 224..231
    slots = paging.slot_mapping(np.array([table]), [0] * L, list(range(L)), bs)
    expect = list(range(112, 128)) + list(range(32, 48)) + list(range(224, 232))
    assert slots.tolist() == expect
    # waste lives only in the last block, and is below one block
    assert paging.wasted_slots(L, bs) == bs - g["tokens_in_last_block"]


@pytest.mark.parametrize("L", [1, 15, 16, 17, 40, 64, 65, 4096, 131072])
def test_waste_bound(L):
    assert 0 <= paging.wasted_slots(L, 16) < 16


def test_gather_follows_logical_order():
    """Rows come back in logical order whatever the physical placement."""
    bs, Hkv, D = 16, 1, 2
    cache = np.zeros((20, bs, Hkv, D), dtype=np.float32)
    table = [7, 2, 14]
    for t in range(40):
        cache[table[t // bs], t % bs, 0, :] = [t, -t]
    rows = paging.gather_sequence(cache, table, 40, bs)
    assert rows[:, 0, 0].tolist() == list(range(40))
    assert rows[:, 0, 1].tolist() == [-t for t in range(40)]


# --------------------------------------------------------------------------
# GQA mapping and scalar counts (KV Cache Engineering, section 1)
# --------------------------------------------------------------------------

def test_gqa_mapping_and_scalars():
    g = golden("gqa_mapping.json")
    for case in g["cases"]:
        m = [attention.kv_head_of(h, g["query_heads"], case["kv_heads"]) for h in range(g["query_heads"])]
        assert m == case["mapping"], case["name"]
        scalars = sizes.kv_cache_bytes(1, case["kv_heads"], g["head_size"], g["tokens"], 1)
        assert scalars == case["cached_scalars"], case["name"]


# --------------------------------------------------------------------------
# sizes
# --------------------------------------------------------------------------

def test_cache_sizes():
    g = golden("cache_sizes.json")
    for c in g["cases"]:
        if c["kind"] == "block":
            assert sizes.block_bytes(c["block_size"], c["kv_heads"], c["head_dim"], c["bytes"]) == c["expect_bytes"]
        elif c["kind"] == "sequence":
            b = sizes.kv_cache_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["tokens"], c["bytes"])
            assert b == c["expect_gib"] * 2 ** 30, c["source"]
        elif c["kind"] == "scalars":
            one = sizes.kv_cache_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["tokens"], 1)
            assert one == c["expect_scalars"]
            assert 2 * one == 2048
        elif c["kind"] == "hybrid_kb":
            for tokens, kb in c["tokens_to_kb"]:
                assert sizes.kv_cache_bytes(1, 1, c["width"], tokens, c["bytes"]) // 1024 == kb
            assert c["width"] * c["width"] * c["bytes"] // 1024 == c["recurrent_kb"]
    p = g["pool"]
    per_tok = sizes.kv_bytes_per_token(80, 8, 128, 2)
    assert per_tok == 320 * 1024
    assert sizes.kv_bytes_per_token(80, 8, 128, 1) == 160 * 1024
    for kib, tokens in p["per_token_kib"]:
        assert sizes.tokens_in_pool(p["pool_bytes"], kib * 1024) == tokens


def test_page_13b_example_is_not_consistent():
    """t13_4 quotes ~800 MB for a 13B FP16 model at 2048 tokens.  With the
    usual 13B attention shape (40 layers, 40 heads of 128) the formula gives
    about 1.6 GiB, so that figure is not used as a pin."""
    b = sizes.kv_cache_bytes(40, 40, 128, 2048, 2)
    assert b / 2 ** 30 > 1.5


# --------------------------------------------------------------------------
# sliding window and StreamingLLM keep-mask
# --------------------------------------------------------------------------

def test_sliding_window_example():
    g = golden("sliding_window.json")
    for pos, expect in enumerate(g["retained_after_token"]):
        assert attention.kept_positions(pos + 1, sink=0, window=g["window"]).tolist() == expect


def test_streaming_llm_layout():
    g = golden("streaming_llm_layout.json")
    L = 131072
    kept = attention.kept_positions(L, g["sink_tokens"], g["window_tokens"])
    assert kept.size == g["total_entries"]
    assert kept[:4].tolist() == [0, 1, 2, 3]
    assert kept[4:].tolist() == list(range(L - 4092, L))
    # short sequences keep every token
    for L in (1, 4, 4095, 4096):
        assert attention.kept_positions(L, 4, 4092).tolist() == list(range(L))
    assert attention.kept_positions(4097, 4, 4092).tolist() == [0, 1, 2, 3] + list(range(5, 4097))


# --------------------------------------------------------------------------
# quantiser (KV Cache Engineering, section 8)
# --------------------------------------------------------------------------

def test_quantizer_4bit_example():
    g = golden("quant4_example.json")
    codes, sc = quant.quantize_int(np.array(g["values"]), g["bits"])
    assert codes.tolist() == g["codes"]
    restored = quant.dequantize(codes, sc)
    assert np.round(restored.astype(np.float64), 3).tolist() == g["restored_3dp"]
    assert len(g["values"]) * 16 == g["payload_bits"][0]
    assert len(g["values"]) * g["bits"] == g["payload_bits"][1]
    # the page's float64 arithmetic gives the same codes
    v = np.array(g["values"])
    s64 = np.max(np.abs(v)) / 7
    assert np.clip(np.rint(v / s64), -7, 7).astype(int).tolist() == g["codes"]


def test_int8_quantizer_properties():
    rng = np.random.default_rng(0)
    for trial in range(50):
        x = (rng.standard_normal((16, 128)) * rng.uniform(0.01, 100)).astype(np.float32)
        codes, sc = quant.quantize_int(x, 8)
        assert sc == np.float32(np.float32(np.abs(x).max()) / np.float32(127))
        i = np.unravel_index(np.abs(x).argmax(), x.shape)
        assert abs(int(codes[i])) == 127 and np.sign(codes[i]) == np.sign(x[i])
        assert codes.min() >= -127 and codes.max() <= 127
        err = np.abs(x.astype(np.float64) - codes * np.float64(sc))
        assert (err <= np.float64(sc) * (0.5 + 2 ** -20)).all()
    codes, sc = quant.quantize_int(np.zeros((16, 128), np.float32), 8)
    assert sc == 0 and (codes == 0).all()


def test_int8_half_even_ties():
    # x/sc lands exactly on .5: 127 * [0.5/127 ...] -- construct ties directly
    x = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5], dtype=np.float32)
    codes, sc = quant.quantize_int(x, 8)
    assert sc == 1.0
    assert codes.tolist() == [127, 0, 2, 2, 0, -2, -2]


# --------------------------------------------------------------------------
# FP8 E4M3 codec against torch's float8_e4m3fn (a library routine)
# --------------------------------------------------------------------------

def test_e4m3_decode_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    ours = codecs.E4M3_TABLE.astype(np.float32)
    nan = np.isnan(t)
    assert (np.isnan(ours) == nan).all()
    assert nan.sum() == 2                       # 0x7F and 0xFF only
    assert (ours[~nan] == t[~nan]).all()
    assert np.signbit(ours[0x80]) and ours[0x80] == 0
    assert codecs.E4M3_TABLE[0x7E] == 448.0
    assert codecs.E4M3_TABLE[0x01] == 2.0 ** -9
    assert codecs.E4M3_TABLE[0x38] == 1.0


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    mags = codecs.E4M3_TABLE[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2           # exact ties
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.01,
        mags, -mags, mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 1000),
        [0.0, -0.0, 2.0 ** -10, -2.0 ** -10, 2.0 ** -11, 448.0, -448.0, 460.0],
    ]).astype(np.float32)
    ours = codecs.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all(), np.nonzero(ours != ref)[0][:10]


def test_e4m3_roundtrip_and_saturation():
    finite = [c for c in range(256) if not np.isnan(codecs.E4M3_TABLE[c])]
    vals = codecs.E4M3_TABLE[finite].astype(np.float32)
    assert codecs.e4m3_encode(vals).tolist() == finite
    assert codecs.e4m3_encode(np.array([465.0, 1e30, -1e30], np.float32)).tolist() == [0x7E, 0x7E, 0xFE]
    assert codecs.e4m3_encode(np.array([-1e-30], np.float32)).tolist() == [0x80]


def test_fp8_quantizer_properties():
    rng = np.random.default_rng(2)
    for trial in range(20):
        x = (rng.standard_normal((16, 128)) * rng.uniform(0.01, 100)).astype(np.float32)
        codes, sc = quant.quantize_fp8(x)
        assert sc == np.float32(np.float32(np.abs(x).max()) / np.float32(448))
        i = np.unravel_index(np.abs(x).argmax(), x.shape)
        assert codes[i] & 0x7F == 0x7E
        restored = codecs.e4m3_to_f32(codes).astype(np.float64) * sc
        # within half an e4m3 ulp of the scaled value's binade (3 mantissa bits)
        y = np.abs(x.astype(np.float64) / sc)
        ulp = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
        assert (np.abs(restored / sc - x / sc) <= ulp / 2 * (1 + 1e-6) + 1e-7).all()


# --------------------------------------------------------------------------
# FP8 E5M2 codec against torch's float8_e5m2 (a library routine)
# --------------------------------------------------------------------------

def test_e5m2_decode_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).float().numpy()
    ours = codecs.E5M2_TABLE.astype(np.float32)
    nan = np.isnan(t)
    assert (np.isnan(ours) == nan).all()
    assert nan.sum() == 6                       # exponent 31 with a nonzero mantissa
    assert (ours[~nan] == t[~nan]).all()        # infinities included
    assert ours[0x7C] == np.inf and ours[0xFC] == -np.inf
    assert codecs.E5M2_TABLE[0x7B] == 57344.0
    assert codecs.E5M2_TABLE[0x01] == 2.0 ** -16
    assert codecs.E5M2_TABLE[0x3C] == 1.0
    # an E5M2 byte is the high byte of the binary16 number of the same value
    f16 = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float32)
    assert (f16[~nan] == ours[~nan]).all()


def test_e5m2_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    mags = codecs.E5M2_TABLE[:0x7C]
    mids = (mags[:-1] + mags[1:]) / 2           # exact ties
    x = np.concatenate([
        rng.uniform(-57344, 57344, 20000),
        rng.standard_normal(20000) * 0.001,
        mags, -mags, mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 1e6),
        [0.0, -0.0, 2.0 ** -17, -2.0 ** -17, 2.0 ** -18, 57344.0, -57344.0],
    ]).astype(np.float32)
    ours = codecs.e5m2_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert (ours == ref).all(), np.nonzero(ours != ref)[0][:10]


def test_e5m2_roundtrip_and_saturation():
    finite = [c for c in range(256) if np.isfinite(codecs.E5M2_TABLE[c])]
    vals = codecs.E5M2_TABLE[finite].astype(np.float32)
    assert codecs.e5m2_encode(vals).tolist() == finite
    # past the largest finite value the quantiser saturates instead of
    # rounding to infinity
    assert codecs.e5m2_encode(np.array([61440.0, 1e30, -1e30], np.float32)).tolist() == [0x7B, 0x7B, 0xFB]
    assert codecs.e5m2_encode(np.array([-1e-30], np.float32)).tolist() == [0x80]


def test_e5m2_quantizer_properties():
    rng = np.random.default_rng(4)
    for trial in range(20):
        x = (rng.standard_normal((16, 128)) * rng.uniform(0.01, 100)).astype(np.float32)
        codes, sc = quant.quantize_fp8(x, "e5m2")
        assert sc == np.float32(np.float32(np.abs(x).max()) / np.float32(57344))
        i = np.unravel_index(np.abs(x).argmax(), x.shape)
        assert codes[i] & 0x7F == 0x7B
        restored = codecs.e5m2_to_f32(codes).astype(np.float64) * sc
        # within half an e5m2 ulp of the scaled value's binade (2 mantissa bits)
        y = np.abs(x.astype(np.float64) / sc)
        ulp = np.where(y < 2.0 ** -14, 2.0 ** -16, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -14))) - 2))
        assert (np.abs(restored / sc - x / sc) <= ulp / 2 * (1 + 1e-6) + 1e-7).all()


def test_bf16_decode_matches_torch():
    x = torch.randn(10000).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert (codecs.bf16_bits_to_f32(bits) == x.float().numpy()).all()
    y = torch.randn(10000).to(torch.float16)
    assert (codecs.f16_bits_to_f32(y.view(torch.int16).numpy().view(np.uint16)) == y.float().numpy()).all()


# --------------------------------------------------------------------------
# pool (KV Cache Engineering, section 10; t13_4 copy-on-write)
# --------------------------------------------------------------------------

def test_paging_free_list_example():
    g = golden("paging_free_list.json")
    p = pool.BlockPool(g["num_blocks"])
    a = p.allocate_sequence(3, 1)
    b = p.allocate_sequence(2, 1)
    assert a == g["request_a"] and b == g["request_b"]
    p.release(a)
    assert list(p.free_list) == g["free_after_a"]
    c = p.allocate_sequence(2, 1)
    assert c == g["request_c"]


def test_append_allocates_exactly_at_block_boundary():
    p = pool.BlockPool(8)
    table = []
    for L in range(0, 50):
        before = len(table)
        slot, cow = p.append(table, L, 16)
        assert cow is None
        assert (len(table) > before) == (L % 16 == 0)
        assert slot == paging.slot_of(table, L, 16)
    assert len(table) == 4


def test_copy_on_write_only_when_shared():
    p = pool.BlockPool(10)
    parent = p.allocate_sequence(40, 16)          # 3 blocks, last partial
    child = p.fork(parent)
    assert p.stats()["shared"] == 3
    slot, cow = p.append(parent, 40, 16)          # shared partial block -> copy
    assert cow is not None and cow[0] == child[2] and parent[2] == cow[1]
    assert p.refcount[cow[0]] == 1 and p.refcount[cow[1]] == 1
    slot2, cow2 = p.append(child, 40, 16)         # no longer shared -> in place
    assert cow2 is None and slot2 == child[2] * 16 + 8
    slot3, cow3 = p.append(parent, 41, 16)
    assert cow3 is None
    with pytest.raises(ValueError):
        p.decref(p.free_list[0])
    q = pool.BlockPool(1)
    q.alloc()
    with pytest.raises(pool.PoolExhausted):
        q.alloc()


# --------------------------------------------------------------------------
# appending to a quantised cache
# --------------------------------------------------------------------------

@pytest.mark.parametrize("code", ["i8", "fp8e4m3", "fp8e5m2", "i4"])
def test_token_by_token_requantisation_ends_at_the_whole_block_codes(code):
    """A block filled one token at a time, quantised again from its tail after
    each token, ends with exactly the codes and scales of quantising the
    whole block at once; in between, every written row is within half a
    step of its source value (INT8) and unwritten rows hold code 0."""
    rng = np.random.default_rng(21)
    tile = rng.standard_normal((16, 2, 32)).astype(np.float32)
    tile[:, 1, 5] *= 8.0
    for rows in range(1, 17):
        codes, scales = quant.requantize_tail(tile, rows, code)
        assert not codes[rows:].any()
        if code == "i8":
            back = quant.dequantize(codecs.decode(codes[:rows], "i8"), scales[None, :, None])
            assert (np.abs(back - tile[:rows]) <= scales[None, :, None] * 0.5 * (1 + 1e-6)).all()
    whole, whole_sc = quant.quantize_cache_blocks(tile[None], code)
    assert codes.tobytes() == whole[0].tobytes()
    assert scales.view(np.uint32).tolist() == whole_sc[0].view(np.uint32).tolist()


def test_page_example_grows_one_value_at_a_time():
    """The section-8 example's six values entered one by one into a 4-bit
    group: the last requantisation prints the page's codes."""
    g = golden("quant4_example.json")
    vals = np.array(g["values"], dtype=np.float32)
    codes = None
    for n in range(1, len(vals) + 1):
        x = np.zeros_like(vals)
        x[:n] = vals[:n]
        codes, sc = quant.quantize_int(x, g["bits"])
    assert codes.tolist() == g["codes"]


# --------------------------------------------------------------------------
# INT4 storage: the page's 4-bit rule, two codes per byte
# --------------------------------------------------------------------------

def test_i4_packing_round_trip_and_layout():
    codes = np.array([[-7, -4, -1, 2, 4, 7, 0, -8]])
    packed = codecs.i4_pack(codes)
    # element 2i in the low nibble, 2i + 1 in the high nibble, two's complement
    assert packed.tolist() == [[0xC9, 0x2F, 0x74, 0x80]]
    assert codecs.i4_unpack(packed).tolist() == codes.tolist()
    every = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)])
    assert (codecs.i4_unpack(codecs.i4_pack(every)) == every).all()


def test_i4_cache_blocks_follow_the_page_example_rule():
    """An INT4 block is the page's 4-bit quantiser over the [16, D] tile,
    packed: decoding and rescaling gives back the rule's restored values."""
    g = golden("quant4_example.json")
    tile = np.zeros((1, 16, 1, 8), dtype=np.float32)
    tile[0, 0, 0, :6] = g["values"]
    codes, scales = quant.quantize_cache_blocks(tile, "i4")
    assert codes.shape == (1, 16, 1, 4)
    vals = codecs.decode(codes, "i4")
    assert vals[0, 0, 0, :6].tolist() == g["codes"]
    back = quant.dequantize(vals[0, 0, 0, :6], scales[0, 0]).astype(np.float64)
    assert np.round(back, 3).tolist() == g["restored_3dp"]
    assert (vals[0, 1:] == 0).all()


# --------------------------------------------------------------------------
# grouped scales (section 8, KIVI paragraph): K per channel, V per token,
# each group inside one block tile
# --------------------------------------------------------------------------

def test_grouped_page_example_as_one_channel_and_as_one_token():
    """The section-8 example's six values form one group either way: as the
    single channel of a [6, 1] tile or as the single token of a [1, 6] tile
    they give the page's codes and restored values."""
    g = golden("quant4_example.json")
    vals = np.array(g["values"], dtype=np.float32)
    c, sc = quant.quantize_grouped(vals[:, None], "i8", "channel")     # 8-bit first: shape only
    assert c.shape == (6, 1) and sc.shape == (1,)
    col = np.zeros((6, 2), np.float32)
    col[:, 0] = vals                                                   # second channel all zero
    c4, sc4 = quant.quantize_grouped(col, "i4", "channel")
    codes = codecs.decode(c4, "i4")[:, 0]
    assert codes.astype(int).tolist() == g["codes"]
    assert sc4[1] == 0 and not codecs.decode(c4, "i4")[:, 1].any()
    restored = quant.dequantize_grouped(codecs.decode(c4, "i4"), sc4, "channel")[:, 0]
    assert np.round(restored.astype(np.float64), 3).tolist() == g["restored_3dp"]
    row = np.zeros((2, 6), np.float32)
    row[1] = vals
    t4, ts4 = quant.quantize_grouped(row, "i4", "token")
    assert codecs.decode(t4, "i4")[1].astype(int).tolist() == g["codes"]
    assert ts4[0] == 0 and ts4[1] == sc4[0]


@pytest.mark.parametrize("code", ["i8", "fp8e4m3", "fp8e5m2", "i4"])
def test_token_groups_are_channel_groups_of_the_transpose(code):
    rng = np.random.default_rng(41)
    t = rng.standard_normal((16, 32)).astype(np.float32) * rng.uniform(0.1, 10, size=(16, 1)).astype(np.float32)
    ct, st = quant.quantize_grouped(t, code, "token")
    cc, sc = quant.quantize_grouped(np.ascontiguousarray(t.T), code, "channel")
    assert (st.view(np.uint32) == sc.view(np.uint32)).all()
    assert (codecs.decode(ct, code) == codecs.decode(cc, code).T).all()


@pytest.mark.parametrize("code,qmax", [("i8", 127), ("i4", 7)])
def test_channel_groups_fit_their_own_range(code, qmax):
    """Each channel's largest magnitude takes the largest code, every value
    is restored within half a step of its own channel's scale, and the
    largest channel scale is the one-scale tile rule's scale."""
    rng = np.random.default_rng(42)
    t = rng.standard_normal((16, 64)).astype(np.float32)
    t[:, 5] *= 8.0
    t[:, 9] *= 0.01
    c, sc = quant.quantize_grouped(t, code, "channel")
    vals = codecs.decode(c, code)
    for d in range(64):
        i = np.abs(t[:, d]).argmax()
        assert abs(vals[i, d]) == qmax
        assert sc[d] == np.float32(np.float32(np.abs(t[:, d]).max()) / np.float32(qmax))
    back = quant.dequantize_grouped(vals, sc, "channel")
    assert (np.abs(back - t) <= sc[None, :] * 0.5 * (1 + 1e-6)).all()
    _, tile_sc = quant.quantize_int(t, 4 if code == "i4" else 8)
    assert sc.max() == tile_sc


def test_channel_groups_shrink_the_error_of_outlier_tiles():
    """With one channel x8 (config 4's outliers), the other channels' worst
    rounding error under per-channel scales is far below the one-scale
    tile's (the page: smaller groups fit their own ranges)."""
    rng = np.random.default_rng(43)
    t = rng.standard_normal((16, 128)).astype(np.float32)
    t[:, 3] *= 8.0
    c, sc = quant.quantize_grouped(t, "i8", "channel")
    err_g = np.abs(quant.dequantize_grouped(codecs.decode(c, "i8"), sc, "channel") - t)
    ct, tsc = quant.quantize_int(t, 8)
    err_t = np.abs(quant.dequantize(ct, tsc) - t)
    others = np.arange(128) != 3
    assert err_g[:, others].max() < err_t[:, others].max() / 4


def test_grouped_decode_reduces_to_tile_decode_when_all_groups_share_the_range():
    """Tiles whose every channel (for K) and every token (for V) reaches the
    same magnitude get group scales equal to the tile scale, the codes of
    the one-scale rule, and the same attention output."""
    rng = np.random.default_rng(44)
    NB, BS, Hkv, D, Hq = 6, 16, 2, 32, 4
    k = rng.uniform(-1, 1, (NB, BS, Hkv, D)).astype(np.float32)
    v = rng.uniform(-1, 1, (NB, BS, Hkv, D)).astype(np.float32)
    k[:, 0] = 2.0                       # every channel reaches 2 in row 0
    v[:, :, :, 0] = -2.0                # every token reaches 2 in channel 0
    kc, kg, kt = quant.quantize_cache_blocks_grouped(k, "i8", "channel")
    vc, vg, vt = quant.quantize_cache_blocks_grouped(v, "i8", "token")
    kc1, ks1 = quant.quantize_cache_blocks(k, "i8")
    vc1, vs1 = quant.quantize_cache_blocks(v, "i8")
    assert (kc == kc1).all() and (vc == vc1).all()
    assert (kg == ks1[:, :, None]).all() and (vg == vs1[:, :, None]).all() and (kt == ks1).all()
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    tables = np.array([[0, 3, 5], [4, 1, 2]], dtype=np.int32)
    lens = [40, 33]
    a = attention.paged_decode_grouped(q, "f32", kc, vc, "i8", tables, lens, BS, 0.2, kg, vg)
    b = attention.paged_decode(q, "f32", kc1, vc1, "i8", tables, lens, BS, 0.2, ks1, vs1)
    assert (a == b).all()


@pytest.mark.parametrize("code", ["i8", "i4"])
@pytest.mark.parametrize("group", ["channel", "token"])
def test_grouped_requantisation_ends_at_the_whole_block(code, group):
    """A block filled one token at a time with grouped scales ends with the
    codes and scales of quantising it whole.  Token groups: appending a row
    never changes an earlier row's codes or scale.  Channel groups: each
    channel's scale is the running absmax of its written rows over the
    largest code."""
    rng = np.random.default_rng(45)
    tile = rng.standard_normal((16, 2, 32)).astype(np.float32)
    tile[:, 0, 7] *= 8.0
    qmax = 127 if code == "i8" else 7
    prev = None
    for rows in range(1, 17):
        codes, gs, ts = quant.requantize_tail_grouped(tile, rows, code, group)
        assert not codecs.decode(codes[rows:], code).any()
        assert (ts == gs.max(axis=1)).all()
        if group == "token":
            assert not gs[:, rows:].any()
            if prev is not None:
                pc, pg = prev
                assert (codecs.decode(codes[:rows - 1], code) == codecs.decode(pc[:rows - 1], code)).all()
                assert (gs[:, :rows - 1] == pg[:, :rows - 1]).all()
        else:
            run_max = np.abs(tile[:rows]).max(axis=0)                         # [Hkv, D]
            assert (gs == (run_max / np.float32(qmax)).astype(np.float32)).all()
        prev = (codes, gs)
    whole, wgs, wts = quant.quantize_cache_blocks_grouped(tile[None], code, group)
    assert codes.tobytes() == whole[0].tobytes()
    assert (gs.view(np.uint32) == wgs[0].view(np.uint32)).all() and (ts == wts[0]).all()
