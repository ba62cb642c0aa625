"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function the public header declares, and its argument checks, names,
error strings and variant choice behave as documented. None of these calls
launches a kernel (argument errors and the M == 0 / N == 0 quick return are
decided before any HIP call; sgemm_f32_plan is host-only by contract)."""
import ctypes
import os
import re

import pytest

import fp32_gemm_tuning_amd as sg
from datagen import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm_f32.h")
PROBE_HEADER = os.path.join(ROOT, "include", "sgemm_f32_probe.h")


def _header_text():
    return open(HEADER).read()


def test_every_declared_function_is_exported():
    text = _header_text() + open(PROBE_HEADER).read()
    names = re.findall(r"SGEMM_F32_API\s+[^;]*?\b(sgemm_f32\w*)\s*\(", text)
    assert len(names) >= 9 and "sgemm_f32_peak_probe" in names
    lib = ctypes.CDLL(sg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in sgemm_f32.h but not exported"


def test_variant_enum_matches_names():
    enum = dict((m.group(1), int(m.group(2))) for m in
                re.finditer(r"SGEMM_F32_(\w+)\s*=\s*(\d+)", _header_text()))
    assert enum["NUM_VARIANTS"] == sg.sgemm_f32_num_variants() == len(sg.VARIANTS)
    for i, name in enumerate(sg.VARIANTS):
        assert sg.sgemm_f32_variant_name(i) == name
        assert sg.sgemm_f32_variant_by_name(name) == i
    assert sg.sgemm_f32_variant_name(-1) is None
    assert sg.sgemm_f32_variant_name(len(sg.VARIANTS)) is None
    assert sg.sgemm_f32_variant_by_name("nope") == -1
    assert enum["MFMA_128"] == sg.VARIANTS.index("mfma_128x128")


@pytest.mark.parametrize("code", [0, -1, -2, -3, -5, -6, -7, -8, -10, -11, -12, -100, -101,
                                  -102, -103, -104, -105, -999])
def test_strerror_is_static_text(code):
    s = sg.sgemm_f32_strerror(code)
    assert isinstance(s, str) and len(s) > 3


# Fake but aligned device addresses: only their alignment is inspected on the
# paths exercised here.
P = 1 << 20


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4), -1),
    ((4, -1, 4, 1.0, P, 4, P, 4, 0.0, P, 4), -2),
    ((4, 4, -1, 1.0, P, 4, P, 4, 0.0, P, 4), -3),
    ((4, 4, 4, 1.0, 0, 4, P, 4, 0.0, P, 4), -5),
    ((4, 4, 4, 1.0, P + 2, 4, P, 4, 0.0, P, 4), -5),
    ((4, 4, 8, 1.0, P, 7, P, 4, 0.0, P, 4), -6),
    ((4, 4, 4, 1.0, P, 4, 0, 4, 0.0, P, 4), -7),
    ((4, 5, 4, 1.0, P, 4, P, 4, 0.0, P, 5), -8),
    ((4, 4, 4, 1.0, P, 4, P, 4, 0.0, 0, 4), -10),
    ((4, 4, 4, 1.0, P, 4, P, 4, 0.0, P + 1, 4), -10),
    ((4, 6, 4, 1.0, P, 4, P, 6, 0.0, P, 5), -11),
    ((0, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 3), -11),   # ld checked even when M == 0
])
def test_argument_errors(args, code):
    assert sg.sgemm_f32(*args, stream=0) == code
    assert sg.sgemm_f32_variant(0, *args, stream=0) == code
    assert sg.sgemm_f32_plan(*args, 256)[0] == code


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4), -1),
    ((4, 4, 4, 1.0, 0, 4, P, 4, 0.0, P, 4), -5),
    ((4, 4, 8, 1.0, P, 7, P, 4, 0.0, P, 4), -6),
    ((4, 4, 4, 1.0, P, 4, P, 4, 0.0, P + 1, 4), -10),
])
def test_ws_static_argument_errors_before_any_hip_call(args, code):
    # The fixed-scratch entry point checks its arguments before it looks up
    # the scratch on a device, so these need no GPU.
    for v in (-1, 7):
        assert sg.sgemm_f32_ws_static(v, sg.ROW_MAJOR, 0, 0, *args, stream=0) == code
    assert sg.sgemm_f32_ws_static(-1, 2, 0, 0, *args, stream=0) == -13
    assert sg.sgemm_f32_ws_static(-1, 0, 2, 0, *args, stream=0) == -14


def test_ws_static_variant_range_and_empty_product():
    args = (4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4)
    assert sg.sgemm_f32_ws_static(-2, 0, 0, 0, *args, stream=0) == sg.ERR_VARIANT
    assert sg.sgemm_f32_ws_static(len(sg.VARIANTS), 0, 0, 0, *args, stream=0) == sg.ERR_VARIANT
    # M == 0 or N == 0: nothing touched, no device needed
    assert sg.sgemm_f32_ws_static(-1, 0, 0, 0, 0, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, stream=0) == 0
    assert sg.sgemm_f32_ws_static(-1, 1, 0, 0, 4, 0, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, stream=0) == 0


def test_scratch_size_matches_header():
    m = re.search(r"#define\s+SGEMM_F32_SCRATCH_BYTES\s+\((\d+)u \* (\d+)u \* (\d+)u\)",
                  _header_text())
    assert m is not None
    assert int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == sg.SCRATCH_BYTES
    m = re.search(r"#define\s+SGEMM_F32_ERR_SCRATCH\s+\((-\d+)\)", _header_text())
    assert int(m.group(1)) == sg.ERR_SCRATCH


def test_unread_operands_may_be_null():
    # M == 0 or N == 0: nothing is read or written, returns 0 without a launch
    assert sg.sgemm_f32(0, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, stream=0) == 0
    assert sg.sgemm_f32(4, 0, 4, 1.0, 0, 4, 0, 1, 0.0, 0, 1, stream=0) == 0
    # K == 0 or alpha == 0: A and B not needed (plan reports the quick return)
    assert sg.sgemm_f32_plan(4, 4, 0, 1.0, 0, 1, 0, 4, 0.5, P, 4, 256) == (0, -1)
    assert sg.sgemm_f32_plan(4, 4, 4, 0.0, 0, 4, 0, 4, 0.5, P, 4, 256) == (0, -1)


def test_bad_variant_id():
    args = (4, 4, 4, 1.0, P, 4, P, 4, 0.0, P, 4)
    assert sg.sgemm_f32_variant(-1, *args, stream=0) == sg.ERR_VARIANT
    assert sg.sgemm_f32_variant(99, *args, stream=0) == sg.ERR_VARIANT


def _plan(M, N, K, lda=None, ldb=None, ldc=None, cus=256, off=0):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    rc, v = sg.sgemm_f32_plan(M, N, K, 1.0, P + off, lda, P, ldb, 0.0, P, ldc, cus)
    assert rc == 0
    return sg.sgemm_f32_variant_name(v)


def test_plan_picks_matrix_core_kernels_for_the_workloads():
    w = WORKLOADS
    assert _plan(4096, 4096, 4096) == "mfma_256x256"
    assert _plan(w["S2048"].M, w["S2048"].N, w["S2048"].K) == "mfma_128x128"
    assert _plan(w["S8192"].M, w["S8192"].N, w["S8192"].K) == "mfma_256x256"
    assert _plan(w["S4092"].M, w["S4092"].N, w["S4092"].K) == "mfma_256x256"
    # 1000 x 1531 is exactly 256 tiles of 64x96: one 12-wave K-split tile per CU
    assert _plan(w["R_odd"].M, w["R_odd"].N, w["R_odd"].K) == "mfma_64x96_kg4"
    assert _plan(w["R_skinny"].M, w["R_skinny"].N, w["R_skinny"].K) == "mfma_skinny"
    assert _plan(256, 256, 256) == "mfma_direct"


def test_plan_busiest_cu_rule():
    # 4096^2: one 256^2 tile per CU (16 waves of one workgroup) beats four
    # 128^2 tiles, eight 64x128 or sixteen 64^2 tiles.
    assert _plan(4096, 4096, 4096, cus=256) == "mfma_256x256"
    # 2048^2: 64 tiles of 256^2 would leave 192 CUs idle; one 128^2 tile each
    # (8 waves of 64x32, 32-deep slices).
    assert _plan(2048, 2048, 2048, cus=256) == "mfma_128x128"
    # 4096 x 2048: 128 tiles of 256^2 (half the CUs) lose to two 128^2 per CU.
    assert _plan(4096, 2048, 4096, cus=256) == "mfma_128x128"
    # 1024x1536: 96 tiles of 128^2 keep 160 CUs idle; 256 tiles of 64x96 do not.
    assert _plan(1024, 1536, 768, cus=256) == "mfma_64x96_kg4"
    # 1000^3: one tile per CU, either 256 tiles of 64^2 or 176 twelve-wave
    # K-group tiles of 96x64 or 64x96 (measured within 0.5% of each other:
    # 35.4-35.6 us), never a kernel that leaves whole rounds of CUs idle.
    assert _plan(1000, 1000, 1000, cus=256) in ("mfma_64x64", "mfma_96x64_kg4", "mfma_64x96_kg4")
    # 8192^2: four rounds of 256^2 tiles.
    assert _plan(8192, 8192, 8192, cus=256) == "mfma_256x256"
    # a single CU: the largest tile always wins.
    assert _plan(1000, 1000, 1000, cus=1) == "mfma_256x256"


def test_plan_direct_kernel_where_its_grid_fits_one_or_two_tiles_per_cu():
    # The direct kernel's 32x32 grid holds one or two tiles per CU (at most
    # 512 tiles): it keeps every CU busy where the 64x64 grid uses a quarter
    # of them (measured per launch: 512^3 10.5 against 13.3 us for
    # mfma_64x64, 512x512x2048 23.9 against 37.7, 576^3 13.6 against 14.5,
    # 600x600x1200 23.3 against 28.0, 1416x324x588 14.7 against 16.8).
    for M, N, K in [(448, 448, 448), (512, 512, 512), (512, 512, 2048), (256, 1024, 1024),
                    (384, 640, 1536), (442, 347, 2477), (576, 576, 576), (704, 704, 704),
                    (600, 600, 1200), (1416, 324, 588)]:
        assert _plan(M, N, K) == "mfma_direct", (M, N, K)
    # three or more tiles per CU, or short K: mfma_64x64 (768^3 17.6 against
    # 23.0 us, 300x2000x300 11.5 against 12.8, 1024x1024x256 7.6 against 13.5
    # back to back).
    for M, N, K in [(1024, 1024, 256), (1000, 1000, 100), (300, 2000, 300), (768, 768, 768),
                    (1024, 1024, 1024)]:
        assert _plan(M, N, K) == "mfma_64x64", (M, N, K)
    # below 64 Mi multiply-adds the direct kernel runs whatever the grid
    assert _plan(1000, 1000, 60) == "mfma_direct"


def test_plan_falls_back_when_offsets_exceed_32_bits():
    # leading dimensions so large that even a 32-row (or 16-row) panel spans
    # more than 2^31 bytes
    assert _plan(256, 256, 16, lda=1 << 26) == "reg2d"
    assert _plan(256, 256, 16, ldb=1 << 26) == "reg2d"
    assert _plan(2048, 2048, 2048, lda=1 << 24) == "reg2d"


def test_peak_probe_argument_checks():
    # rejected before any launch
    assert sg.sgemm_f32_peak_probe(7, 1, 1, P)[0] == -1
    assert sg.sgemm_f32_peak_probe(0, 0, 1, P)[0] == -2
    assert sg.sgemm_f32_peak_probe(0, 1, 0, P)[0] == -3
    assert sg.sgemm_f32_peak_probe(0, 1, 1, 0)[0] == -4
