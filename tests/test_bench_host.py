"""Host logic of bench.py (CPU): the algorithmic byte model of an attention
launch and the rule that counter summaries count only for the source they
were taken on."""
import os

import pytest

import bench
from patch_attention_cfg_amd import inputs


@pytest.mark.parametrize("name,mb", [
    ("sdxl1024-64x64", 26.21),   # Q + O + K + V, bf16
    ("sdxl1024-32x32", 13.11),
    ("sdxl2048", 94.37),
    ("sdxl3840", 331.78),
    ("dit1024", 132.12),
])
def test_attention_bytes_without_landing(name, mb):
    lv = inputs.LEVELS[name]
    e = 2
    want = 2 * lv.B * lv.H * lv.n * lv.d * e + 2 * lv.B * lv.H * lv.N_kv * lv.d * e
    got = bench.attention_bytes(lv, False)
    assert got == want
    assert abs(got / 1e6 - mb) < 0.01


def test_landing_adds_the_fresh_rows_write():
    for name in ("sdxl1024-64x64", "dit1024"):
        lv = inputs.LEVELS[name]
        extra = bench.attention_bytes(lv, True) - bench.attention_bytes(lv, False)
        assert extra == 2 * lv.B * lv.H * (lv.n + lv.n_text) * lv.d * 2


def test_small_level_roofline_is_bandwidth_bound():
    lv = inputs.LEVELS["sdxl1024-32x32"]
    ai = lv.flops() / bench.attention_bytes(lv, True)
    assert ai * bench.PEAK_HBM_GBPS / 1e3 < bench.PEAK_BF16_TFLOPS   # below the ridge
    lv = inputs.LEVELS["sdxl3840"]
    ai = lv.flops() / bench.attention_bytes(lv, False)
    assert ai * bench.PEAK_HBM_GBPS / 1e3 > bench.PEAK_BF16_TFLOPS


def test_counted_follows_the_source_hash(tmp_path):
    src = "patch_attention_cfg_amd/csrc/cfg_step.hip"
    good = tmp_path / "good.txt"
    good.write_text(f"# header: not a field\nsource_sha256: {bench.source_sha(src)}\nread_bytes: 42\n")
    assert bench.counted(str(good), src, "read_bytes") == 42.0
    assert bench.counted(str(good), src, "missing") is None
    stale = tmp_path / "stale.txt"
    stale.write_text("source_sha256: 0000\nread_bytes: 42\n")
    assert bench.counted(str(stale), src, "read_bytes") is None
    assert bench.counted(str(tmp_path / "absent.txt"), src, "read_bytes") is None


def test_committed_summaries_match_the_committed_sources():
    """Every committed counter summary names the kernel source it was taken
    on; the headline ones must match the sources as committed, or the
    benchmark would report their figures as null."""
    prof = os.path.join(bench.ROOT, "profiles")
    pairs = [("attn_bf16_sdxl3840_hbm_traffic.txt", "attention_bf16.hip"),
             ("attn_bf16_sdxl3840_sq_counters.txt", "attention_bf16.hip"),
             ("cfg_step_sdxl3840_hbm_traffic.txt", "cfg_step.hip")]
    for fname, src in pairs:
        f = bench.profile_fields(os.path.join(prof, fname))
        assert f.get("source_sha256") == bench.source_sha(
            f"patch_attention_cfg_amd/csrc/{src}"), fname
