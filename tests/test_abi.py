"""The C-ABI library loads on a machine without a GPU, exports every entry
point include/mxfp4.h declares, and rejects bad arguments on the host before
any HIP call (so no GPU is needed for these checks)."""
import ctypes
import os
import re

import pytest

import block_scaled_mxfp4_bf16_amd as mx
import synthetic as syn
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mxfp4.h")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp4_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(mx.exported_symbols())


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(mx.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_library_exports_nothing_else():
    out = os.popen("nm -D --defined-only %s" % mx.LIB_PATH).read()
    names = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    ours = {n for n in names if n.startswith("mxfp4")}
    assert ours == set(declared_functions())


def test_size_helpers():
    assert mx.mxfp4_packed_bytes(16, 1536) == 16 * 768
    assert mx.mxfp4_raw_scale_bytes(16, 1536) == 16 * 48
    assert mx.mxfp4_shuffled_scale_bytes(2112, 7168) == 2304 * 224
    assert mx.mxfp4_shuffled_scale_bytes(3072, 1536) == 3072 * 48
    assert mx.mxfp4_shuffled_scale_bytes(16, 96) == 256 * 8
    assert mx.mxfp4_packed_bytes(0, 64) == 0


def test_status_strings():
    L = mx.lib()
    for code in range(5):
        assert L.mxfp4_status_string(code).startswith(b"MXFP4")


FAKE = 1 << 20  # an aligned non-null address; never dereferenced (checks fail first)


@pytest.mark.parametrize("args,code", [
    ((0, FAKE, FAKE, FAKE, 16, 64, 128), INVALID),           # null A
    ((FAKE, FAKE, FAKE, 0, 16, 64, 128), INVALID),           # null C
    ((FAKE, FAKE, FAKE, FAKE, 0, 64, 128), INVALID),         # M = 0
    ((FAKE, FAKE, FAKE, FAKE, 16, -32, 128), INVALID),       # N < 0
    ((FAKE + 8, FAKE, FAKE, FAKE, 16, 64, 128), INVALID),    # misaligned A
    ((FAKE, FAKE, FAKE, FAKE, 16, 64, 96), UNSUPPORTED),     # K % 64 != 0
    ((FAKE, FAKE, FAKE, FAKE, 16, 48, 128), UNSUPPORTED),    # N % 32 != 0
    ((FAKE, FAKE, FAKE, FAKE, 1 << 16, 64, 1 << 15), UNSUPPORTED),  # A beyond 2^31 bytes
])
def test_gemm_rejects_bad_arguments(args, code):
    L = mx.lib()
    assert L.mxfp4_gemm(*args, None) == code
    assert L.mxfp4_gemm_ex(*args, None, 0, None) == code
    assert L.mxfp4_gemm_noalloc(*args, None) == code


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """The no-allocation entry point checks the chosen schedule's workspace
    against its fixed scratch size on the host, before any HIP call."""
    L = mx.lib()
    limit = 8 * 1024 * 1024
    M, N, K = 4096, 4096, 8192  # large-M kernel: its quantized A operand alone is ~17 MB
    assert mx.mxfp4_gemm_workspace_bytes(M, N, K) > limit
    assert L.mxfp4_gemm_noalloc(FAKE, FAKE, FAKE, FAKE, M, N, K, None) == WORKSPACE
    # the benchmark shapes all fit
    for w in list(syn.CONFIGS.values()) + list(syn.EXTRA_SHAPES.values()):
        assert mx.mxfp4_gemm_workspace_bytes(w.M, w.N, w.K) <= limit, w.name


def test_gemm_ex_rejects_small_workspace():
    L = mx.lib()
    M, N, K = 16, 2112, 7168
    need = mx.mxfp4_gemm_workspace_bytes(M, N, K)
    assert need > 0  # long K at small M: this shape's schedule splits K over workgroups
    assert L.mxfp4_gemm_ex(FAKE, FAKE, FAKE, FAKE, M, N, K, None, 0, None) == WORKSPACE
    assert L.mxfp4_gemm_ex(FAKE, FAKE, FAKE, FAKE, M, N, K, FAKE, need - 1, None) == WORKSPACE
    assert L.mxfp4_gemm_ex(FAKE, FAKE, FAKE, FAKE, M, N, K, FAKE + 16, need, None) == WORKSPACE


@pytest.mark.parametrize("args,code", [
    ((0, 16, 64, FAKE, FAKE, 0), INVALID),
    ((FAKE, 0, 64, FAKE, FAKE, 0), INVALID),
    ((FAKE, 16, 16, FAKE, FAKE, 0), INVALID),
    ((FAKE, 16, 48, FAKE, FAKE, 0), UNSUPPORTED),
    ((FAKE + 4, 16, 64, FAKE, FAKE, 0), INVALID),
])
def test_quantize_rejects_bad_arguments(args, code):
    assert mx.lib().mxfp4_quantize(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((FAKE, FAKE, 24, 64, FAKE, FAKE), UNSUPPORTED),
    ((FAKE, FAKE, 32, 48, FAKE, FAKE), UNSUPPORTED),
    ((FAKE, 0, 32, 64, FAKE, FAKE), INVALID),
])
def test_preshuffle_rejects_bad_arguments(args, code):
    assert mx.lib().mxfp4_preshuffle_b(*args, None) == code


@pytest.mark.parametrize("args,code", [
    ((0, 32, 64, FAKE, FAKE), INVALID),
    ((FAKE, 0, 64, FAKE, FAKE), INVALID),
    ((FAKE, 32, 16, FAKE, FAKE), INVALID),
    ((FAKE + 8, 32, 64, FAKE, FAKE), INVALID),
    ((FAKE, 24, 64, FAKE, FAKE), UNSUPPORTED),
    ((FAKE, 32, 48, FAKE, FAKE), UNSUPPORTED),
    ((FAKE, 1 << 16, 1 << 15, FAKE, FAKE), UNSUPPORTED),
])
def test_prepare_b_rejects_bad_arguments(args, code):
    assert mx.lib().mxfp4_prepare_b(*args, None) == code


def test_gemm_q_rejects_bad_arguments_and_names_pre_quantized_schedules():
    L = mx.lib()
    assert L.mxfp4_gemm_q(FAKE, None, FAKE, FAKE, FAKE, 16, 64, 128, None) == INVALID
    assert L.mxfp4_gemm_q(None, FAKE, FAKE, FAKE, FAKE, 16, 64, 128, None) == INVALID
    assert L.mxfp4_gemm_q(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 64, 96, None) == UNSUPPORTED
    assert L.mxfp4_gemm_q(FAKE + 8, FAKE, FAKE, FAKE, FAKE, 16, 64, 128, None) == INVALID
    for shape in ((1, 64, 128), (8, 2112, 7168), (16, 3072, 1536), (32, 4096, 512), (64, 7168, 2048)):
        assert mx.mxfp4_gemm_q_schedule_name(*shape).endswith("_pq"), shape
    assert mx.mxfp4_gemm_q_schedule_name(256, 7168, 7168).startswith("wide_")
    # an override that reads bf16 A cannot serve pre-quantized A
    mx.mxfp4_set_schedule_override("mt1_nt1_wn2_wk4_kpw1_split3")
    try:
        assert mx.mxfp4_gemm_q_schedule_name(16, 3072, 1536) is None
    finally:
        mx.mxfp4_set_schedule_override(None)


def test_schedule_names_and_override():
    name = mx.mxfp4_gemm_schedule_name(16, 3072, 1536)
    assert re.fullmatch(r"mt\d+_nt\d+_wn\d+_wk\d+_kpw\d+_split\d+", name)
    assert mx.mxfp4_gemm_schedule_name(16, 3072, 96) is None
    with pytest.raises(RuntimeError):
        mx.mxfp4_set_schedule_override("mt9_nt9_wn9_wk9_kpw9_split1")
    mx.mxfp4_set_schedule_override("mt1_nt1_wn2_wk4_kpw1_split3")
    try:
        assert mx.mxfp4_gemm_schedule_name(16, 3072, 1536) == "mt1_nt1_wn2_wk4_kpw1_split3"
        # an override that cannot cover K: the shape is unsupported under it
        assert mx.mxfp4_gemm_schedule_name(16, 3072, 7168 * 4) is None
    finally:
        mx.mxfp4_set_schedule_override(None)
    assert mx.mxfp4_gemm_schedule_name(16, 3072, 1536) == name


def test_eight_row_schedules_only_cover_m_up_to_8():
    mx.mxfp4_set_schedule_override("mt1_nt1_wn1_wk16_kpw4_split1_r8")
    try:
        assert mx.mxfp4_gemm_schedule_name(8, 2112, 7168) == "mt1_nt1_wn1_wk16_kpw4_split1_r8"
        assert mx.mxfp4_gemm_schedule_name(1, 256, 512) == "mt1_nt1_wn1_wk16_kpw4_split1_r8"
        assert mx.mxfp4_gemm_schedule_name(9, 2112, 7168) is None
    finally:
        mx.mxfp4_set_schedule_override(None)
    # without an override, small M picks an 8-row schedule unless tuned otherwise
    assert mx.mxfp4_gemm_schedule_name(4, 512, 1024).endswith("_r8")
    assert not mx.mxfp4_gemm_schedule_name(9, 512, 1024).endswith("_r8")


def test_wide_schedule_names():
    assert mx.mxfp4_gemm_schedule_name(256, 7168, 7168).startswith("wide_")
    mx.mxfp4_set_schedule_override("wide_mt4_nt7_w8_d2_split2")
    try:
        assert mx.mxfp4_gemm_schedule_name(256, 7168, 7168) == "wide_mt4_nt7_w8_d2_split2"
        assert mx.mxfp4_gemm_schedule_name(256, 7168 - 32, 7168) is None  # N not a multiple of 112
    finally:
        mx.mxfp4_set_schedule_override(None)
    # B staged through LDS: named only, never the default
    mx.mxfp4_set_schedule_override("widel_mt4_nt7_w4_d4_split1")
    try:
        assert mx.mxfp4_gemm_schedule_name(256, 7168, 7168) == "widel_mt4_nt7_w4_d4_split1"
    finally:
        mx.mxfp4_set_schedule_override(None)
    for M, N, K in ((256, 7168, 7168), (128, 2048, 4096), (1024, 7168, 2048)):
        assert not mx.mxfp4_gemm_schedule_name(M, N, K).startswith("widel_")
    for bad in ("wide_mt4_nt7_w8_d9_split1", "wide_mt3_nt7_w8_d2_split1", "wide_mt4_nt7_w8_d2_split1_pq", "wide_mt4_nt7_d2_split1",
                "widel_mt4_nt7_w8_d2_split1", "widel_mt4_nt7_w4_d4_split1_r8", "widl_mt4_nt7_w4_d4_split1"):
        with pytest.raises(RuntimeError):
            mx.mxfp4_set_schedule_override(bad)


def test_quant_mode_knob():
    with pytest.raises(RuntimeError):
        mx.mxfp4_set_quant_mode(2)
    mx.mxfp4_set_quant_mode(1)
    mx.mxfp4_set_quant_mode(0)


def test_every_schedule_the_gpu_tests_name_covers_its_shape():
    """The GPU tests force schedules by name; each must resolve for the
    shape it is used with (checked here so that a typo fails on the CPU)."""
    from tests import test_gpu_gemm as g
    cases = [(s, M, N, K) for s, M, N, K in g.WIDE_CASES]
    cases += [(s, M, 256, 2048 + 64) for s in g.R8_SCHEDULES for M in (1, 5, 8)]
    cases += [(s, 70, 224, 1088) for s in g.RAGGED_SCHEDULES]
    cases += [(s, M, N, K) for s, M, N, K in g.GEMM_Q_CASES]
    cases += [(s, M, N, K) for s, M, N, K in g.STREAMK_CASES + g.ATOMIC_CASES]
    try:
        for s in g.SCHEDULES:  # compiled (the test skips those that cannot cover its K)
            mx.mxfp4_set_schedule_override(s)
        for s, M, N, K in cases:
            mx.mxfp4_set_schedule_override(s)
            assert mx.mxfp4_gemm_schedule_name(M, N, K) == s, (s, M, N, K)
    finally:
        mx.mxfp4_set_schedule_override(None)


def test_split_epilogue_schedule_names_cover_and_size():
    """Float-atomic ("_at") and stream-K ("streamk<G>") schedules: accepted
    only in their own name forms, never picked by default, refused where a
    workgroup's run would exceed its K capacity or the grid exceeds the
    iterations, and sized as their layouts say."""
    # 40x256x2112, 32-column tiles: 24 tiles x 17 steps = 408 iterations;
    # one workgroup covers wk*kpw = 32 steps; a tile holds 16x32 f32
    M, N, K = 40, 256, 2112
    e = 16 * 32 * 4
    try:
        mx.mxfp4_set_schedule_override("mt1_nt2_wn1_wk8_kpw4_streamk13")
        assert mx.mxfp4_gemm_schedule_name(M, N, K) == "mt1_nt2_wn1_wk8_kpw4_streamk13"
        assert mx.mxfp4_gemm_workspace_bytes(M, N, K) == 65536 + 13 * 2 * e
        mx.mxfp4_set_schedule_override("mt1_nt2_wn1_wk8_kpw4_streamk12")  # runs of 34 > 32 steps
        assert mx.mxfp4_gemm_schedule_name(M, N, K) is None
        mx.mxfp4_set_schedule_override("mt1_nt2_wn1_wk8_kpw4_streamk409")  # more workgroups than iterations
        assert mx.mxfp4_gemm_schedule_name(M, N, K) is None
        mx.mxfp4_set_schedule_override("mt1_nt2_wn1_wk8_kpw4_streamk408")
        assert mx.mxfp4_gemm_schedule_name(M, N, K) == "mt1_nt2_wn1_wk8_kpw4_streamk408"
        mx.mxfp4_set_schedule_override("mt1_nt2_wn1_wk8_kpw4_split3_at")
        assert mx.mxfp4_gemm_schedule_name(M, N, K) == "mt1_nt2_wn1_wk8_kpw4_split3_at"
        assert mx.mxfp4_gemm_workspace_bytes(M, N, K) == 65536 + 24 * e  # one f32 tile per output tile
        mx.mxfp4_set_schedule_override("mt1_nt2_wn1_wk8_kpw4_split3")
        assert mx.mxfp4_gemm_workspace_bytes(M, N, K) == 65536 + 24 * 3 * e
        mx.mxfp4_set_schedule_override("mt1_nt2_wn1_wk8_kpw4_streamk50_r8")
        assert mx.mxfp4_gemm_schedule_name(5, N, K) == "mt1_nt2_wn1_wk8_kpw4_streamk50_r8"
        assert mx.mxfp4_gemm_schedule_name(9, N, K) is None  # 8-row staging is for M <= 8
    finally:
        mx.mxfp4_set_schedule_override(None)
    for bad in ("mt1_nt2_wn1_wk8_kpw4_split3_pq_at", "mt1_nt2_wn1_wk8_kpw4_split3_at_r8",
                "mt1_nt2_wn1_wk8_kpw4_streamk13_at", "mt1_nt2_wn1_wk8_kpw4_streamk13_pq",
                "mt1_nt2_wn1_wk8_kpw4_streamk0", "mt2_nt2_wn1_wk8_kpw4_streamk13", "mt1_nt2_wn1_wk8_kpw3_split3_at"):
        with pytest.raises(RuntimeError):
            mx.mxfp4_set_schedule_override(bad)
    for shape in ((40, 256, 2112), (8, 2112, 7168), (16, 2112, 7168), (16, 3072, 1536), (64, 7168, 2048)):
        name = mx.mxfp4_gemm_schedule_name(*shape)
        assert "streamk" not in name and not name.endswith("_at"), (shape, name)


def test_k_too_long_for_the_fused_kernels_goes_to_the_large_m_kernel():
    # 16 splits of the deepest 16-row fused kernel (14 waves x 4 steps of 128)
    # cover K = 16 * 56 * 128 = 114688
    assert not mx.mxfp4_gemm_schedule_name(16, 64, 114688).startswith("wide_")
    assert mx.mxfp4_gemm_schedule_name(16, 64, 114688 + 128).startswith("wide_")
    for M in (1, 16, 64):
        assert mx.mxfp4_gemm_schedule_name(M, 64, 262144).startswith("wide_")
        assert mx.mxfp4_gemm_q_schedule_name(M, 64, 262144).startswith("wide_")
    # the largest operands the ABI takes still have a schedule
    assert mx.mxfp4_gemm_schedule_name(32767, 32, 32768) is not None
    assert mx.mxfp4_gemm_schedule_name(32767, 32736, 64) is not None


@pytest.mark.parametrize("M,N,K,q", [(32, 4096, 512, False), (8, 2112, 7168, False), (256, 7168, 7168, False),
                                     (100, 224, 2112, False), (32, 4096, 512, True), (1, 64, 64, False)])
def test_listed_schedules_round_trip_and_include_the_builtin(M, N, K, q):
    names = mx.mxfp4_list_schedules(M, N, K, q)
    assert names and len(names) == len(set(names))
    builtin = (mx.mxfp4_gemm_q_schedule_name if q else mx.mxfp4_gemm_schedule_name)(M, N, K)
    assert builtin in names
    ks = (K + 127) // 128
    step = max(1, len(names) // 60)  # a spread of them: each is accepted and serves the shape as named
    try:
        for n in names[::step] + names[-3:]:
            assert int(n.rsplit("split", 1)[1].split("_")[0]) <= ks
            mx.mxfp4_set_schedule_override(n)
            assert (mx.mxfp4_gemm_q_schedule_name if q else mx.mxfp4_gemm_schedule_name)(M, N, K) == n
    finally:
        mx.mxfp4_set_schedule_override(None)


def test_list_schedules_sizing_and_rejected_shapes():
    L = mx.lib()
    need = L.mxfp4_list_schedules(16, 3072, 1536, 0, None, 0)
    full = ctypes.create_string_buffer(need + 1)
    assert L.mxfp4_list_schedules(16, 3072, 1536, 0, full, need + 1) == need
    assert len(full.value) == need and full.value.endswith(b"\n")
    small = ctypes.create_string_buffer(11)
    assert L.mxfp4_list_schedules(16, 3072, 1536, 0, small, 11) == need
    assert small.value == full.value[:10]  # cut at the cap, NUL-terminated
    for shape in ((0, 64, 64), (16, 48, 64), (16, 64, 96), (16, 64, 0)):
        assert L.mxfp4_list_schedules(*shape, 0, None, 0) == 0
        assert mx.mxfp4_list_schedules(*shape) == []


def test_above_64_rows_the_choice_compares_kernel_families():
    # the large-M kernel wins on long enough K and wide N; a fused kernel on short K or narrow N
    assert mx.mxfp4_gemm_schedule_name(192, 2048, 4096).startswith("wide_")
    assert mx.mxfp4_gemm_schedule_name(128, 14336, 4096) == "wide_mt4_nt7_w4_d2_split1"
    assert not mx.mxfp4_gemm_schedule_name(129, 3584, 2048).startswith("wide")
    assert not mx.mxfp4_gemm_schedule_name(160, 5120, 1024).startswith("wide")
    # 256-column fused tiles only where their steps cover K exactly
    assert mx.mxfp4_gemm_schedule_name(32, 8192, 8192) == "mt1_nt2_wn8_wk2_kpw8_split4"
    assert "_wn8_" not in mx.mxfp4_gemm_schedule_name(160, 5120, 1024)
    assert "_wn8_" not in mx.mxfp4_gemm_schedule_name(64, 4096, 14336)
    # below 64 rows it competes too: long K and wide N
    assert mx.mxfp4_gemm_schedule_name(64, 4096, 14336).startswith("wide_")
    assert not mx.mxfp4_gemm_schedule_name(16, 4096, 14336).startswith("wide")
    # the large-M kernel does not split K across workgroups unless K is beyond the fused kernels
    for M, N, K in ((96, 7168, 2048), (192, 2048, 7168), (256, 4096, 4096), (128, 4096, 14336)):
        name = mx.mxfp4_gemm_schedule_name(M, N, K)
        assert not name.startswith("wide") or name.endswith("_split1"), name
