"""Register budget: no kernel instance the automatic choice can launch spills.

The pages' rule is that the best per-thread tile is the largest one that does
not spill ("100 Days of GPU, Day 44", "Solution" and "Pitfalls"). The build
saves the compiler's per-kernel resource remarks to _build/resource_usage.txt
(fp32_gemm_tuning_amd/build.py). For every instance whose scratch size is
not zero, this test works out which variant and which form (16-byte,
register-staged or 4-byte fill; whole tiles or masked; transpositions) it is,
builds a call that takes exactly that form, installs a one-entry dispatch
model holding that variant, and checks that sgemm_f32_plan_ws does not
choose it. Every other kernel (the skinny and direct kernels, the
fallbacks, the stream-K fix-up) must not spill at all. A positive control
checks that spill-free forms are still chosen.
"""
import os
import re
import subprocess

import pytest

import fp32_gemm_tuning_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REMARKS = os.path.join(ROOT, "_build", "resource_usage.txt")
CUS = 256
WS = 1 << 40
P = 1 << 20       # fake, 16-byte aligned device address (plans read no memory)

PIPE = {(256, 256): "mfma_256x256", (128, 128): "mfma_128x128", (64, 128): "mfma_64x128",
        (64, 64): "mfma_64x64"}
KGROUP = {(64, 128): "mfma_64x128_kg4", (64, 96): "mfma_64x96_kg4", (96, 64): "mfma_96x64_kg4",
          (128, 128): "mfma_128x128_kg4"}


def instances():
    """(demangled kernel name, scratch bytes per lane) for every kernel of the build."""
    if not os.path.exists(REMARKS):
        pytest.fail(f"{REMARKS} is missing: build the library first (fp32_gemm_tuning_amd/build.py)")
    names, scratch = [], []
    for line in open(REMARKS):
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            names.append(m.group(1))
            scratch.append(None)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and names:
            scratch[-1] = int(m.group(1))
    dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                         check=True).stdout.splitlines()
    assert len(dem) == len(names) and all(s is not None for s in scratch)
    return list(zip(dem, scratch))


def parse(name):
    """(variant, form) of a model kernel instance, else None. form: dict with
    fill ('vec', 'u16', 'dma4'), full (bool), ta, tb."""
    m = re.match(r"void sgemm::k_mfma_pipe(_sk)?<(\d+), (\d+), \d+, \d+, (\d+), \d+, \d+, "
                 r"(true|false), (true|false), (true|false), (true|false)(, (true|false))?>", name)
    if m:
        sk, bm, bn, bk = m.group(1), int(m.group(2)), int(m.group(3)), int(m.group(4))
        vec, full, ta, tb = (m.group(i) == "true" for i in range(5, 9))
        u16 = m.group(10) == "true"
        v = PIPE[(bm, bn)] + ("_sk" if sk else "")
        fill = "vec" if vec else "u16" if u16 else "dma4"
        return v, dict(fill=fill, full=full, ta=ta, tb=tb, bm=bm, bn=bn, bk=bk)
    m = re.match(r"void sgemm::k_mfma_kgroup<(\d+), (\d+), \d+, \d+, (\d+), (\d), "
                 r"(true|false), (true|false)>", name)
    if m:
        bm, bn, bk, fill = int(m.group(1)), int(m.group(2)), int(m.group(3)), int(m.group(4))
        ta, tb = m.group(5) == "true", m.group(6) == "true"
        return KGROUP[(bm, bn)], dict(fill={0: "dma4", 1: "u16", 2: "vec"}[fill], full=False,
                                      ta=ta, tb=tb, bm=bm, bn=bn, bk=bk)
    return None


def call_for(variant, form):
    """Row-major (M, N, K, lda, ldb, ldc, transa, transb) that takes `form`
    of `variant` under a one-entry model: enough tiles to fill the unit
    count, split for a stream-K kernel (tiles not a multiple of 256)."""
    bm, bn, bk = form["bm"], form["bn"], form["bk"]
    ta, tb = form["ta"], form["tb"]
    tm, tn = (16, 19) if variant.endswith("_sk") else (16, 16)
    M, N = tm * bm, tn * bn
    K = 64 * bk
    if form["fill"] == "dma4":
        K = 3                       # a contiguous extent below 4: no 16-byte fill at all
        M, N = 64 * bm, 64 * bn     # keeps the product out of the tiny-shape path
        if variant.endswith("_sk"):
            N += bn                 # 64 x 65 tiles: not a multiple of the units
    if not form["full"] and variant in PIPE.values() or variant.endswith("_sk") and not form["full"]:
        M += 4                      # a partial tile row (keeps every extent a multiple of 4)
    # stored extents: A is M x K (K x M if ta), B is K x N (N x K if tb)
    a_cols = M if ta else K
    b_cols = K if tb else N
    lda, ldb = a_cols, b_cols
    if form["fill"] in ("dma4", "u16"):
        lda += 1                    # odd leading dimension: no 16-byte chunks
    return M, N, K, lda, ldb, N, int(ta), int(tb)


def plan_with_only(variant, M, N, K, lda, ldb, ldc, ta, tb):
    entry = {"variant": variant, "overhead_us": 0.0, "eff": [1.0, 1.0, 1.0, 1.0], "fill4": 1.0,
             "tile_us": 0.0}
    assert sg.sgemm_f32_set_model([entry]) == 0
    try:
        rc, v = sg.sgemm_f32_plan_ws(sg.ROW_MAJOR, ta, tb, M, N, K, 1.0, P, lda, P, ldb, 0.0, P,
                                     ldc, WS, CUS)
    finally:
        sg.sgemm_f32_set_model([])
    assert rc == 0, sg.sgemm_f32_strerror(rc)
    return sg.sgemm_f32_variant_name(v)


def test_remarks_cover_the_kernels():
    names = [n for n, _ in instances()]
    for key in ("k_mfma_pipe<256, 256", "k_mfma_pipe_sk<128, 128", "k_mfma_kgroup<64, 96",
                "k_mfma_skinny", "k_mfma_direct", "k_sk_fixup"):
        assert any(key in n for n in names), key


def test_no_spilling_instance_is_chosen_automatically():
    spilling = [(n, s) for n, s in instances() if s > 0]
    for name, scratch in spilling:
        parsed = parse(name)
        assert parsed is not None, (
            f"{name} spills {scratch} B/lane and is not a dispatch-model kernel: "
            "the automatic choice or a fallback may launch it")
        variant, form = parsed
        args = call_for(variant, form)
        got = plan_with_only(variant, *args)
        assert got != variant, (f"{name} spills {scratch} B/lane, yet the automatic choice "
                                f"takes it for {args}")


@pytest.mark.parametrize("variant,form", [
    ("mfma_256x256", dict(fill="vec", full=True, ta=False, tb=False)),
    ("mfma_256x256", dict(fill="vec", full=False, ta=True, tb=True)),
    ("mfma_128x128_sk", dict(fill="vec", full=False, ta=False, tb=False)),
    ("mfma_64x96_kg4", dict(fill="u16", full=False, ta=False, tb=False)),
    ("mfma_128x128_kg4", dict(fill="vec", full=False, ta=True, tb=False)),
    ("mfma_128x128", dict(fill="u16", full=False, ta=False, tb=False)),
    ("mfma_64x64", dict(fill="u16", full=False, ta=True, tb=True)),
])
def test_spill_free_forms_are_still_chosen(variant, form):
    bm, bn, bk = sg.sgemm_f32_variant_tile(sg.sgemm_f32_variant_by_name(variant))[1:]
    form = dict(form, bm=bm, bn=bn, bk=bk)
    args = call_for(variant, form)
    assert plan_with_only(variant, *args) == variant, args
