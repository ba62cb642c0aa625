"""The compile-time autotuner's host side: the search spaces, the validity
rules, macro flags, names, and the reading of the compiler's resource report.
(Building copies takes minutes and timing them needs the GPU; neither runs
here.)"""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _autotune():
    spec = importlib.util.spec_from_file_location(
        "autotune", os.path.join(ROOT, "fp32_gemm_tuning_amd", "autotune.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


at = _autotune()
CSRC = os.path.join(ROOT, "fp32_gemm_tuning_amd", "csrc")


def _space_source(space):
    # The space's source file and the header every matrix-core source
    # includes (where the macros a space sets are defined).
    return (open(os.path.join(CSRC, at.SPACES[space]["source"])).read() +
            open(os.path.join(CSRC, "mfma_common.hpp")).read())


@pytest.mark.parametrize("space", sorted(at.SPACES))
def test_first_configuration_is_the_in_tree_build(space):
    # Every macro a space sets exists in the kernel source with the first
    # value of its list as the default, so configuration 0 is the control.
    c = at.configs(space)[0]
    src = _space_source(space)
    for macro, value in c.items():
        assert f"#define {macro} {value}\n" in src, macro


@pytest.mark.parametrize("space", sorted(at.SPACES))
def test_configurations_are_unique_and_valid(space):
    cs = at.configs(space)
    names = [at.config_name(space, c) for c in cs]
    assert len(set(names)) == len(names) > 0
    for c in cs:
        assert at._valid(space, c)
        assert at.flags(c) == [f"-D{k}={v}" for k, v in c.items()]


def test_tile_rules():
    base = at.configs("tile")[0]

    def with_(**kw):
        c = dict(base)
        c.update({"SGEMM_M128_" + k: v for k, v in kw.items()})
        return at._valid("tile", c)

    assert with_()
    assert not with_(WM=48)                        # wave tile not whole 32x32 blocks
    assert not with_(BM=96, WM=64)                 # wave tile does not divide the block
    assert not with_(BM=256, BN=256, WM=32, WN=32)  # 64 waves > 16 per workgroup
    assert not with_(BM=256, BN=128, WM=32, WN=64, WAVES_PER_EU=2)  # 16 waves need 4 per SIMD
    assert not with_(BM=256, BN=256, BK=64)        # LDS: 2 x 128 KB > 160 KB
    assert not with_(WM=128, WN=128)               # 256 accumulators leave no room at 4 waves
    # pipe: LDS per stage counts
    p = at.configs("pipe")[0]
    assert at._valid("pipe", p)
    assert not at._valid("pipe", dict(p, SGEMM_M256_BK=32, SGEMM_M256_STAGES=3))  # 192 KB


def test_resource_report_parsing():
    text = "\n".join([
        "remark: x: Function Name: _ZN5sgemm11k_mfma_pipeILi128ELi128ELi64ELi32ELi32ELi2ELi4ELb1ELb1E",
        "remark: x:     VGPRs: 92",
        "remark: x:     ScratchSize [bytes/lane]: 0",
        "remark: x: Function Name: _ZN5sgemm11k_mfma_pipeILi128ELi128ELi64ELi32ELi32ELi2ELi3ELb0ELb0E",
        "remark: x:     VGPRs: 134",
        "remark: x:     ScratchSize [bytes/lane]: 12",
        "remark: x: Function Name: _ZN5sgemm11k_mfma_pipeILi256ELi256ELi64ELi64ELi16ELi2ELi4ELb1ELb1E",
        "remark: x:     VGPRs: 128",
        "remark: x:     ScratchSize [bytes/lane]: 64",
    ])
    tile0, pipe0 = at.configs("tile")[0], at.configs("pipe")[0]
    assert at._resources(text, at.kernel_pattern("tile", tile0)) == {"vgpr": 134, "scratch": 12}
    assert at._resources(text, at.kernel_pattern("pipe", pipe0)) == {"vgpr": 128, "scratch": 64}
    assert at._resources(text, "k_mfma_kgroup") == {"vgpr": 0, "scratch": 0}


@pytest.mark.parametrize("space", sorted(at.SPACES))
def test_kernel_pattern_names_the_configured_instance(space):
    # Each configuration's pattern is a fragment of an Itanium-mangled name
    # with that configuration's tile sizes.
    for c in at.configs(space):
        pat = at.kernel_pattern(space, c)
        assert "{" not in pat and pat.startswith("k_mfma_")


def test_shapes_argument():
    assert at._shapes("4096x4096x4096,1000x1531x777") == [(4096, 4096, 4096), (1000, 1531, 777)]
