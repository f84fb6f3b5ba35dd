"""The C ABI without a GPU: the library loads, exports every declared
symbol, rejects bad schemes and shapes at load, and the planner follows its
rules. No call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from quantized_moe_align_amd import qma

ROOT_DIR = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "qma.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qma.LIB_PATH):
        pytest.skip("libqma.so not built")
    return qma.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qma_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_symbols()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(qma.EXPORTS)


def test_version_and_status_strings(L):
    assert "gfx950" in qma.qma_version()
    assert qma._status_name(qma.QMA_ERR_UNSUPPORTED) == "QMA_ERR_UNSUPPORTED"


@pytest.mark.parametrize("field,value", [
    ("weight_bits", 8), ("zero_point", 0), ("group_size", 64), ("group_size", 128),
    ("scale_dtype", qma.DTYPE_FP16), ("scale_dtype", qma.DTYPE_FP32),
    ("act_dtype", qma.DTYPE_FP16), ("pack_format", 2)])
def test_unsupported_schemes_fail_at_load(L, field, value):
    with pytest.raises(qma.QmaError) as ei:
        qma.qma_layer_create(8, 256, 256, qma.PATH_INDEXED, qma.w4a16_desc(**{field: value}))
    assert ei.value.status == qma.QMA_ERR_UNSUPPORTED
    assert field.split("_")[0] in ei.value.detail or "only" in ei.value.detail


@pytest.mark.parametrize("E,N,K", [(0, 256, 256), (8, 24, 256), (8, 256, 96), (8, 256, 200),
                                   (8, 0, 256)])
def test_bad_shapes(L, E, N, K):
    with pytest.raises(qma.QmaError) as ei:
        qma.qma_layer_create(E, N, K)
    assert ei.value.status == qma.QMA_ERR_INVALID_ARG


def test_fused_activation_layer_rules(L):
    F = qma.LAYER_FUSE_SILU_MUL
    # unknown flag bits and widths that cannot pair gate and up tiles per wave
    for N, flags in ((4096, 2), (4096, F | 4), (4064, F), (96, F)):
        with pytest.raises(qma.QmaError) as ei:
            qma.qma_layer_create(8, N, 1024, flags=flags)
        assert ei.value.status == qma.QMA_ERR_INVALID_ARG, (N, flags)
    lay = qma.qma_layer_create(48, 4096, 7168, flags=F)
    try:
        # the planner's plans give every wave gate/up pairs
        for T in (12, 576, 48 * 40, 8192):
            p = qma.qma_plan_indexed(lay, T, 1, 0)
            if p.kernel == qma.KERNEL_SMALL_M:
                assert (p.block_n // (16 * (4 // p.waves_k))) % 2 == 0, T
        # the same packed size as the unfused layer (only the tile order differs)
        plain = qma.qma_layer_create(48, 4096, 7168)
        assert qma.qma_packed_weight_bytes(plain) == qma.qma_packed_weight_bytes(lay)
        qma.qma_layer_destroy(plain)
        # host checks before any launch: one tile per wave, and the
        # producer/consumer kernel, have no fused epilogue
        fake = 1 << 20                     # rejected on the host; never dereferenced
        p = qma.qma_plan_indexed(lay, 12, 1, 16)
        p.block_n, p.waves_k, p.split_k, p.schedule = 16, 4, 1, 0
        with pytest.raises(qma.QmaError) as ei:
            qma.qma_indexed_gemm(lay, p, fake, 12, 1, fake, fake, fake, fake, 12 + 15, 12,
                                 None, fake, stream=0)
        assert ei.value.status == qma.QMA_ERR_INVALID_ARG and "even" in ei.value.detail
        q = qma.qma_plan_indexed(lay, 48 * 100, 1, 128)
        q.kernel, q.split_k = qma.KERNEL_LARGE_M_PC, 1
        with pytest.raises(qma.QmaError) as ei:
            qma.qma_indexed_gemm(lay, q, fake, 4800, 1, fake, fake, fake, fake, 4800 + 48 * 127,
                                 4800, None, fake, stream=0)
        assert ei.value.status == qma.QMA_ERR_INVALID_ARG and "fused" in ei.value.detail
    finally:
        qma.qma_layer_destroy(lay)


def test_per_expert_weights_must_fit_32_bit_offsets(L):
    # kernels address one expert's packed blocks with 32-bit offsets: N x K / 2
    # bytes of nibbles must stay below 2 GiB (65536 x 65536 / 2 = 2 GiB exactly)
    with pytest.raises(qma.QmaError) as ei:
        qma.qma_layer_create(1, 65536, 65536)
    assert ei.value.status == qma.QMA_ERR_INVALID_ARG and "2 GiB" in ei.value.detail
    lay = qma.qma_layer_create(1, 65536 - 16, 65536)      # one tile less fits
    qma.qma_layer_destroy(lay)


def test_null_out_pointer(L):
    d = qma.w4a16_desc()
    assert L.qma_layer_create(ctypes.byref(d), 8, 256, 256, 0, None) == qma.QMA_ERR_INVALID_ARG


@pytest.mark.parametrize("E,N,K,profile", [
    (48, 4096, 7168, "ep_gate_up"), (48, 7168, 2048, "ep_down"),
    (384, 512, 7168, "tp_gate_up"), (384, 7168, 256, "tp_down"),
    (8, 256, 256, "ep_gate_up"), (8, 256, 128, "ep_down")])
def test_profile_inferred_from_shape(L, E, N, K, profile):
    lay = qma.qma_layer_create(E, N, K)
    try:
        info = qma.qma_layer_info(lay)
        assert info["profile"] == profile and (info["E"], info["N"], info["K"]) == (E, N, K)
        # uint4 + one bf16 scale per 32 values = 0.5625 bytes per weight
        assert qma.qma_packed_weight_bytes(lay) == E * N * K * 9 // 16
    finally:
        qma.qma_layer_destroy(lay)


def _plan(E, N, K, T, topk, force=0):
    lay = qma.qma_layer_create(E, N, K)
    try:
        return qma.qma_plan_indexed(lay, T, topk, force)
    finally:
        qma.qma_layer_destroy(lay)


def test_plan_decode_ep8():
    p = _plan(48, 4096, 7168, 576, 1)
    assert p.kernel == qma.KERNEL_SMALL_M and p.block_m == 16
    # 48 tiles x 16 blocks of 256 columns: one full round of three per CU
    assert p.block_n == 256 and p.waves_k == 1 and p.split_k == 1
    assert p.k_depth == 256                            # shared-row kernel: 2 chunks
    assert p.schedule == qma.SCHEDULE_GANG and p.est_tiles == 768
    # EP16 share: at 256 columns only 384 workgroups, so 128 columns
    q = _plan(24, 4096, 7168, 288, 1)
    assert q.block_m == 16 and q.block_n == 128 and q.waves_k == 1
    assert q.schedule == qma.SCHEDULE_GANG and q.est_tiles == 768
    assert p.tok_e_x100 == 1200 and p.rows == 576
    assert qma.qma_workspace_bytes(p) == 0


def test_plan_tp8_and_tiny():
    p = _plan(384, 512, 7168, 256, 8)
    assert p.block_m == 16 and p.tok_e_x100 == 533 and p.split_k == 1
    # 384 x 2 items of 256 columns fill one round of the gang schedule
    assert p.waves_k == 1 and p.block_n == 256 and p.schedule == qma.SCHEDULE_GANG
    t = _plan(8, 256, 256, 64, 2)
    assert t.block_m == 16 and t.waves_k == 1          # waves side by side on columns
    assert t.block_n == 128                            # short K: 256 wide, 8 tiles -> narrower
    assert t.split_k == 1                              # K = 256: no room to split
    d = _plan(48, 7168, 2048, 576, 1)                  # EP8 down: K = 2048
    assert d.waves_k == 1 and d.block_n == 128 and d.split_k == 1
    assert d.schedule == qma.SCHEDULE_SEMI_STATIC      # 2688 items: several rounds
    m = _plan(48, 4096, 7168, 48 * 32, 1)              # 32-row tiles: 256 columns
    assert m.block_m == 32 and m.waves_k == 1 and m.block_n == 256
    big = _plan(48, 4096, 7168, 48 * 64, 1)            # 64-row tiles: shared rows, 128 wide
    assert big.block_m == 64 and big.waves_k == 1 and big.block_n == 128 and big.split_k == 1


def test_block_m_follows_tok_e():
    for tok_e, bm in [(1, 16), (15, 16), (16, 16), (17, 32), (32, 32), (33, 64), (79, 64)]:
        assert _plan(48, 4096, 7168, 48 * tok_e, 1).block_m == bm, tok_e


def test_split_k_gate_turns_on_only_when_underfilled():
    # 1 expert: 32 tiles at 128 columns, under two per CU -> split toward
    # three workgroups per CU, capped at 56 / 14 = 4 K runs of 14 chunks
    p = _plan(1, 4096, 7168, 12, 1)
    assert p.block_n == 128 and p.est_tiles == 32 and p.split_k == 4 and p.waves_k == 1
    assert qma.qma_workspace_bytes(p) == p.split_k * 12 * 4096 * 4
    # EP128 share (3 experts): gate_up 96 tiles -> split 4; down (K = 16
    # chunks) has no room for two runs of 14 -> unsplit, 64 columns with
    # the waves on K for twice the workgroups
    g = _plan(3, 4096, 7168, 35, 1)
    assert g.block_n == 128 and g.est_tiles == 96 and g.split_k == 4
    d = _plan(3, 7168, 2048, 35, 1)
    assert d.block_n == 64 and d.waves_k == 4 and d.est_tiles == 336 and d.split_k == 1
    # 8 experts: 256 tiles -> split 3 (768 items, one gang round)
    e8 = _plan(8, 4096, 7168, 96, 1)
    assert e8.split_k == 3 and e8.schedule == qma.SCHEDULE_GANG
    # EP32 share: 12 experts x 32 tiles = 384 -> split 2 on the shared-row
    # kernel, one gang round of 768 items
    q = _plan(12, 4096, 7168, 144, 1)
    assert q.split_k == 2 and q.block_n == 128 and q.waves_k == 1 and q.k_depth == 256
    assert q.schedule == qma.SCHEDULE_GANG
    # 512 tiles and more (two per CU): no split
    assert _plan(16, 4096, 7168, 192, 1).split_k == 1
    # EP32 down (672 tiles) and EP16 gate_up (768 tiles): four waves side by side
    d = _plan(12, 7168, 2048, 144, 1)
    assert d.split_k == 1 and d.block_n == 128 and d.waves_k == 1
    g = _plan(24, 4096, 7168, 288, 1)
    assert g.split_k == 1 and g.block_n == 128 and g.waves_k == 1


def test_stream_rule():
    # TP8 down share: K = 256 is two chunks, so a workgroup streams 7 column
    # blocks (14 chunks) and the grid keeps >= 4 workgroups per CU
    d = _plan(384, 7168, 256, 256, 8)
    assert d.kernel == qma.KERNEL_SMALL_M and d.waves_k == 1 and d.split_k == 1
    assert d.n_stream == 7
    # fewer tiles: the stream shortens until the grid holds 4 workgroups per
    # CU, and no further
    for E, T in ((96, 64), (48, 32), (16, 16)):
        p = _plan(E, 7168, 256, T, 8)
        nb = 7168 // p.block_n
        tiles_m = p.est_tiles // nb
        ns = p.n_stream
        wgs = lambda k: tiles_m * -(-nb // k)
        assert 1 <= ns <= 7
        assert ns == 1 or wgs(ns) >= 4 * 256
        assert ns == 7 or wgs(ns + 1) < 4 * 256
    assert _plan(48, 7168, 2048, 558, 1).n_stream == 1      # EP8 down: K long enough
    assert _plan(48, 4096, 7168, 558, 1).n_stream == 1      # K split across waves
    assert _plan(8, 256, 128, 64, 2).n_stream == 1          # grid too small to stream


def test_gang_schedule_plan_rules():
    # taken where the items fill 5/6 to all of one round of 3 x 256 groups
    for E, T, gang in [(48, 576, True), (40, 480, True), (39, 468, False), (49, 588, False),
                       (24, 288, True), (19, 228, False)]:
        p = _plan(E, 4096, 7168, T, 1)
        assert (p.schedule == qma.SCHEDULE_GANG) == gang, (E, p.est_tiles)
    # never for short K, streaming, K split across waves, split-K or large-M
    assert _plan(384, 7168, 256, 256, 8).schedule == qma.SCHEDULE_SEMI_STATIC
    # 3 experts: split 4 gives 384 items, half a round
    assert _plan(3, 4096, 7168, 36, 1).schedule == qma.SCHEDULE_SEMI_STATIC
    assert _plan(48, 4096, 7168, 48 * 100, 1).schedule == qma.SCHEDULE_SEMI_STATIC
    # 12 tiles folded into 24 column-block groups: 3 x 28 items per XCD
    assert _plan(12, 7168, 2048, 144, 1).schedule == qma.SCHEDULE_GANG
    # masked decode (32-row tiles): 48 x 16 items
    lay = qma.qma_layer_create(48, 4096, 7168, qma.PATH_GROUPED_MASKED)
    try:
        m = qma.qma_plan_grouped(lay, 64, 32)
    finally:
        qma.qma_layer_destroy(lay)
    assert m.block_m == 32 and m.block_n == 256 and m.schedule == qma.SCHEDULE_GANG
    assert qma.qma_workspace_bytes(m) == 0


def test_stream_k_schedule_rules():
    from quantized_moe_align_amd import moe as moe_mod
    fake = 1 << 20                                        # never dereferenced
    lay = qma.qma_layer_create(48, 7168, 2048)
    try:
        p = qma.qma_plan_indexed(lay, 280, 2, 16)
        assert p.block_m == 16 and p.waves_k == 1 and p.split_k == 1
        p.schedule = qma.SCHEDULE_STREAM_K
        assert qma.qma_workspace_bytes(p) == 0
        assert moe_mod.schedule_applies(p, qma.SCHEDULE_STREAM_K)
        bad = []
        for field, value in (("split_k", 2), ("block_m", 64), ("waves_k", 4), ("n_stream", 2)):
            q = qma.qma_plan_indexed(lay, 280, 2, 16)
            setattr(q, field, value)
            if field == "waves_k":
                q.block_n = 64
            q.schedule = qma.SCHEDULE_STREAM_K
            assert not moe_mod.schedule_applies(q, qma.SCHEDULE_STREAM_K), field
            with pytest.raises(qma.QmaError) as ei:
                qma.qma_indexed_gemm(lay, q, fake, 280, 2, fake, fake, fake, fake,
                                     560 + 48 * 63, 560, None, fake, stream=0)
            bad.append(ei.value.status == qma.QMA_ERR_INVALID_ARG)
        assert all(bad)
        # a sorted capacity that could give a group items of three token tiles
        with pytest.raises(qma.QmaError) as ei:
            qma.qma_indexed_gemm(lay, p, fake, 280, 2, fake, fake, fake, fake, 1 << 16, 560,
                                 None, fake, stream=0)
        assert ei.value.status == qma.QMA_ERR_INVALID_ARG and "stream-K" in str(ei.value)
    finally:
        qma.qma_layer_destroy(lay)
    # indexed layers only; short K (fewer than 8 chunks) refused
    m = qma.qma_layer_create(48, 7168, 2048, qma.PATH_GROUPED_MASKED)
    try:
        q = qma.qma_plan_grouped(m, 64, 32)
        q.schedule = qma.SCHEDULE_STREAM_K
        assert not moe_mod.schedule_applies(q, qma.SCHEDULE_STREAM_K)
        with pytest.raises(qma.QmaError) as ei:
            qma.qma_grouped_masked_gemm(m, q, fake, fake, 64, 32, fake, fake, stream=0)
        assert ei.value.status == qma.QMA_ERR_INVALID_ARG
    finally:
        qma.qma_layer_destroy(m)
    short = qma.qma_layer_create(8, 7168, 512)
    try:
        q = qma.qma_plan_indexed(short, 64, 2, 16)
        q.schedule, q.n_stream, q.block_n = qma.SCHEDULE_STREAM_K, 1, 128
        with pytest.raises(qma.QmaError) as ei:
            qma.qma_indexed_gemm(short, q, fake, 64, 2, fake, fake, fake, fake, 128 + 8 * 15,
                                 128, None, fake, stream=0)
        assert ei.value.status == qma.QMA_ERR_INVALID_ARG
    finally:
        qma.qma_layer_destroy(short)


def test_dynamic_schedule_plan_rules():
    p = _plan(48, 4096, 7168, 576, 1)
    p.schedule = qma.SCHEDULE_SEMI_STATIC
    assert qma.qma_workspace_bytes(p) == 0
    p.schedule = qma.SCHEDULE_DYNAMIC
    assert qma.qma_workspace_bytes(p) == 256           # the work counter
    q = _plan(1, 4096, 7168, 12, 1)                    # split-K plan
    q.schedule = qma.SCHEDULE_DYNAMIC
    assert qma.qma_workspace_bytes(q) == q.split_k * 12 * 4096 * 4 + 256


def test_large_m_rule():
    # indexed: large-M from 80 routed rows per expert, or on request
    assert _plan(48, 4096, 7168, 48 * 80, 1).kernel == qma.KERNEL_LARGE_M
    assert _plan(48, 4096, 7168, 48 * 79, 1).kernel == qma.KERNEL_SMALL_M
    p = _plan(8, 256, 256, 64, 2, force=128)
    assert p.kernel == qma.KERNEL_LARGE_M and p.block_m == 128 and p.block_n == 256
    # the producer/consumer form is never planned, split or not
    assert p.split_k == 1                               # K = 256: no room to split
    q = _plan(1, 4096, 7168, 200, 1, force=128)        # 32 tiles: split-K on
    assert q.split_k > 1 and q.kernel == qma.KERNEL_LARGE_M
    # contiguous: every 128-row tile holds one expert, so large-M whatever M/E
    lay = qma.qma_layer_create(48, 4096, 7168, qma.PATH_GROUPED_CONTIGUOUS)
    try:
        for M in (128, 512, 6144):
            q = qma.qma_plan_grouped(lay, M, 0)
            assert q.kernel == qma.KERNEL_LARGE_M and q.block_m == 128, M
    finally:
        qma.qma_layer_destroy(lay)


def test_plan_rejects_bad_force_and_wrong_path():
    for bad in (48, 256):
        with pytest.raises(qma.QmaError):
            _plan(48, 4096, 7168, 576, 1, force=bad)
    with pytest.raises(qma.QmaError):
        _plan(8, 24 * 16, 256, 64, 2, force=128)             # N % 256 != 0
    lay = qma.qma_layer_create(8, 256, 256, qma.PATH_GROUPED_MASKED)
    try:
        with pytest.raises(qma.QmaError):
            qma.qma_plan_indexed(lay, 64, 2)
        p = qma.qma_plan_grouped(lay, 64, 32)
        assert p.block_m == 32 and p.rows == 8 * 64
        with pytest.raises(qma.QmaError):
            qma.qma_plan_grouped(lay, 64, 65)
    finally:
        qma.qma_layer_destroy(lay)


def test_align_sizes_closed_form():
    assert qma.qma_align_sizes(64, 2, 8, 16) == (128 + 8 * 15, (128 + 120 + 15) // 16)
    assert qma.qma_align_sizes(0, 1, 4, 64) == (4 * 63, 4)
    with pytest.raises(qma.QmaError):
        qma.qma_align_sizes(-1, 1, 4, 16)


def test_host_checks_before_any_launch(L):
    # every case below must be rejected on the host, before a kernel launch
    lay = qma.qma_layer_create(8, 256, 256)
    other = qma.qma_layer_create(8, 512, 256)
    try:
        p = qma.qma_plan_indexed(lay, 64, 2)
        cap = qma.qma_align_sizes(64, 2, 8, p.block_m)[0]
        fake = 1 << 20                                   # never dereferenced
        with pytest.raises(qma.QmaError) as e1:           # null c
            qma.qma_indexed_gemm(lay, p, fake, 64, 2, fake, fake, fake, fake, cap, 128,
                                 None, None, stream=0)
        assert e1.value.status == qma.QMA_ERR_INVALID_ARG
        with pytest.raises(qma.QmaError) as e2:           # plan from another layer
            qma.qma_indexed_gemm(other, p, fake, 64, 2, fake, fake, fake, fake, cap, 128,
                                 None, fake, stream=0)
        assert e2.value.status == qma.QMA_ERR_INVALID_ARG
        with pytest.raises(qma.QmaError) as e3:           # too few activation rows
            qma.qma_indexed_gemm(lay, p, fake, 10, 2, fake, fake, fake, fake, cap, 128,
                                 None, fake, stream=0)
        assert e3.value.status == qma.QMA_ERR_INVALID_ARG
        p.split_k = 2                                      # needs a workspace now
        with pytest.raises(qma.QmaError) as e4:
            qma.qma_indexed_gemm(lay, p, fake, 64, 2, fake, fake, fake, fake, cap, 128,
                                 None, fake, None, 0, stream=0)
        assert e4.value.status == qma.QMA_ERR_WORKSPACE
        with pytest.raises(qma.QmaError) as e5:           # capacity below the bound
            qma.qma_moe_align(fake, 64, 2, 8, 16, fake, fake, fake, cap - 1, stream=0)
        assert e5.value.status == qma.QMA_ERR_INVALID_ARG
        with pytest.raises(qma.QmaError) as e6:           # too many experts
            qma.qma_moe_align(fake, 4, 1, 2048, 16, fake, fake, fake, 4 + 2048 * 15, stream=0)
        assert e6.value.status == qma.QMA_ERR_INVALID_ARG
        with pytest.raises(qma.QmaError) as e7:           # misaligned packed weights
            qma.qma_prepack(lay, fake, fake, fake + 4, stream=0)
        assert e7.value.status == qma.QMA_ERR_INVALID_ARG
        p0 = qma.qma_plan_indexed(lay, 64, 2)            # unsplit: no workspace
        with pytest.raises(qma.QmaError) as e9:           # 2 GiB of activations
            qma.qma_indexed_gemm(lay, p0, fake, 1 << 22, 2, fake, fake, fake, fake, cap, 128,
                                 None, fake, stream=0)
        assert e9.value.status == qma.QMA_ERR_INVALID_ARG
        with pytest.raises(qma.QmaError) as e10:          # grid beyond 2^24 workgroups
            qma.qma_indexed_gemm(lay, p0, fake, 64, 2, fake, fake, fake, fake, 1 << 30, 128,
                                 None, fake, stream=0)
        assert e10.value.status == qma.QMA_ERR_INVALID_ARG
        with pytest.raises(qma.QmaError) as e11:          # GEMM capacity below the bound
            qma.qma_indexed_gemm(lay, p0, fake, 64, 2, fake, fake, fake, fake, cap - 1, 128,
                                 None, fake, stream=0)
        assert e11.value.status == qma.QMA_ERR_INVALID_ARG and "bound" in e11.value.detail
        # a large-M plan on K = 256 (two chunks of 128) edited to three K
        # splits: one split would own no chunk, so the host rejects it
        big = qma.qma_plan_indexed(lay, 64, 2, 128)
        assert big.kernel == qma.KERNEL_LARGE_M
        for split in (3, 8):
            big.split_k = split
            with pytest.raises(qma.QmaError) as e12:
                qma.qma_indexed_gemm(lay, big, fake, 64, 2, fake, fake, fake, fake, 1 << 12, 128,
                                     None, fake, fake, 1 << 30, stream=0)
            assert e12.value.status == qma.QMA_ERR_INVALID_ARG and "split_k" in e12.value.detail
        pc = qma.qma_plan_indexed(lay, 64, 2, 128)
        pc.kernel, pc.split_k = qma.KERNEL_LARGE_M_PC, 2      # no split-K in this form
        with pytest.raises(qma.QmaError) as e13:
            qma.qma_indexed_gemm(lay, pc, fake, 64, 2, fake, fake, fake, fake, 1 << 12, 128,
                                 None, fake, fake, 1 << 30, stream=0)
        assert e13.value.status == qma.QMA_ERR_INVALID_ARG
        # edited plans naming no kernel instance: 8 column tiles per wave,
        # waves_k 3, 16 accumulator tiles per wave, 8 with rows held per wave,
        # a streamed 64-column block
        for edit in ({"block_m": 16, "block_n": 128, "waves_k": 4, "split_k": 1},
                     {"block_m": 16, "block_n": 128, "waves_k": 3, "split_k": 1},
                     {"block_m": 64, "block_n": 256, "waves_k": 1, "split_k": 1},
                     {"block_m": 64, "block_n": 128, "waves_k": 2, "split_k": 1},
                     {"block_m": 32, "block_n": 64, "waves_k": 4, "split_k": 1},
                     {"block_m": 16, "block_n": 64, "waves_k": 1, "split_k": 1, "n_stream": 2}):
            q = qma.Plan.from_buffer_copy(qma.qma_plan_indexed(lay, 64, 2))
            for k, v in edit.items():
                setattr(q, k, v)
            with pytest.raises(qma.QmaError) as e8:
                qma.qma_indexed_gemm(lay, q, fake, 64, 2, fake, fake, fake, fake, cap, 128,
                                     None, fake, stream=0)
            assert e8.value.status == qma.QMA_ERR_INVALID_ARG, edit
    finally:
        qma.qma_layer_destroy(lay)
        qma.qma_layer_destroy(other)


def test_missing_library_fails_loudly():
    # no CPU fallback: without the built HIP library every entry point raises
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from quantized_moe_align_amd import qma\n"
        "qma.LIB_PATH = '/nonexistent/libqma.so'\n"
        "try:\n"
        "    qma.qma_layer_create(8, 256, 256)\n"
        "except ImportError as e:\n"
        "    print('raised', e)\n"
        "else:\n"
        "    print('no error')\n" % ROOT_DIR)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert "raised" in r.stdout and "not built" in r.stdout, r.stdout + r.stderr


def xcd_fold(tiles, nblocks):
    """The launch's fold of few token tiles into column-block groups dealt
    to the 8 XCDs: the smallest f in (1, 2, 4, 8) dividing nblocks that fills
    the XCDs to within 10 % of even (written out here from that rule)."""
    if tiles <= 0:
        return 1
    for f in (1, 2, 4, 8):
        if nblocks % f:
            break
        v = tiles * f
        if -(-v // 8) * 8 * 10 <= v * 11:
            return f
    f = 8
    while f > 1 and nblocks % f:
        f //= 2
    return f


def test_xcd_fold_rule():
    assert xcd_fold(3, 32) == 8 and xcd_fold(3, 56) == 8      # EP128: 24 groups
    assert xcd_fold(12, 56) == 2 and xcd_fold(24, 28) == 1    # EP32, EP16
    assert xcd_fold(48, 16) == 1 and xcd_fold(384, 2) == 1    # EP8, TP8
    assert xcd_fold(3, 28) == 4                               # 4 divides 28, 8 does not
    assert xcd_fold(5, 7) == 1                                # nothing divides 7


def test_planner_invariants_over_shapes():
    # every plan the planner returns names an existing kernel instance and
    # follows the documented rules, over a grid of layer and batch shapes
    import itertools
    for E, N, K, T, topk in itertools.product((1, 8, 48, 384), (80, 256, 512, 1040, 4096, 7168),
                                              (256, 2048, 7168), (1, 17, 256, 8192), (1, 8)):
        lay = qma.qma_layer_create(E, N, K)
        try:
            p = qma.qma_plan_indexed(lay, T, topk, 0)
        finally:
            qma.qma_layer_destroy(lay)
        shape = (E, N, K, T, topk)
        assert N % p.block_n == 0, shape
        assert 1 <= p.split_k <= 8 and p.waves_k in (1, 2, 4) and p.n_stream >= 1, shape
        if p.kernel == qma.KERNEL_LARGE_M:
            assert p.block_m == 128 and p.block_n == 256 and N % 256 == 0, shape
            assert T * topk / E >= 80, shape
        else:
            assert p.kernel == qma.KERNEL_SMALL_M and p.block_m in (16, 32, 64), shape
            tm, ntw = p.block_m // 16, p.block_n // (16 * (4 // p.waves_k))
            assert ntw in (1, 2, 4), shape
            # a compiled instance: shared rows (waves_k 1, 2 or 4 column tiles
            # per wave, at most 8 accumulator tiles) or rows per wave (at most 4)
            shared = p.waves_k == 1 and ntw in (2, 4) and tm * ntw <= 8
            assert shared or tm * ntw <= 4, shape
            if p.n_stream > 1:                               # streaming: short K only
                assert K // 128 < 8 and p.block_m == 16 and p.split_k == 1, shape
            if p.schedule == qma.SCHEDULE_GANG:
                # a shared-row instance with long K, one round of groups
                assert shared and p.n_stream == 1 and K // 128 >= 8, shape
                nb = N // p.block_n
                tiles_m = p.est_tiles // nb
                assert 640 <= p.est_tiles * p.split_k <= 768, shape
                f = xcd_fold(tiles_m, nb)
                assert -(-tiles_m * f // 8) * (nb // f) * p.split_k <= 96, shape
            else:
                assert p.schedule == qma.SCHEDULE_SEMI_STATIC, shape
        if p.split_k > 1:
            # split-K only under two workgroups per CU (small-M; large-M
            # under one), and never below 14 128-wide K chunks per split
            # (four for large-M)
            assert p.est_tiles < (256 if p.kernel == qma.KERNEL_LARGE_M else 512), shape
            per_split = 4 if p.kernel == qma.KERNEL_LARGE_M else 14
            assert K // 128 >= per_split * p.split_k, shape
            assert qma.qma_workspace_bytes(p) > 0, shape
        else:
            assert qma.qma_workspace_bytes(p) == 0, shape


def _sk_fits(num_tiles, nblocks, kc, groups, cus=256):
    # the host's bound for the stream-K schedule (a group's range of units
    # touches at most two token tiles), written out from its definition
    per_wg = -(-(num_tiles * nblocks) // cus)
    per_group = -(-(per_wg * kc) // groups)
    span = 1 + -(-(per_group - 1) // kc)
    return span - 1 <= nblocks


def test_stream_k_work_division_model():
    """The stream-K schedule's work division, walked unit by unit as each
    group of a CU walks it: every K chunk of every item is accumulated once,
    the pieces of an item cut between groups meet at the group holding its
    first chunk in K order, and no group meets a third token tile whenever
    the host's bound admits the shape. Brute force over random shapes."""
    import random
    rng = random.Random(7)
    cases = [(48, 56, 16, 4), (3, 56, 16, 4), (1, 1, 8, 4), (5, 2, 8, 3), (384, 56, 2, 4)]
    cases += [(rng.randint(1, 300), rng.randint(1, 60), rng.randint(8, 56), rng.choice([3, 4]))
              for _ in range(150)]
    checked = 0
    for ntiles, nbl, kc, S in cases:
        if not _sk_fits(ntiles, nbl, kc, S):
            continue
        checked += 1
        items, grid = ntiles * nbl, 256
        pieces = {}
        for b in range(grid):
            rk = (b & 7) * (grid >> 3) + (b >> 3)
            i0, i1 = items * rk // grid, items * (rk + 1) // grid
            if i0 >= i1:
                continue
            U = (i1 - i0) * kc
            starts = [U * k // S for k in range(S + 1)]
            for g in range(S):
                ua, ub = starts[g], starts[g + 1]
                assert ub - ua >= 2
                tiles = {(i0 + u // kc) // nbl for u in range(ua, ub)}
                assert max(tiles) - min(tiles) <= 1, (ntiles, nbl, kc, S, b, g)
                for u in range(ua, ub):
                    pieces.setdefault(i0 + u // kc, []).append((g, u % kc))
        assert sorted(pieces) == list(range(items))
        for item, units in pieces.items():
            # every chunk once, the groups in ascending order along K
            assert [c for _, c in units] == list(range(kc)), item
            gs = [g for g, _ in units]
            assert gs == sorted(gs), item
    assert checked > 100
