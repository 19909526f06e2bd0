"""Host checks of the profile summariser: every kernel the library launches
falls in the launch group its call belongs to, and recorded traffic is keyed
by the hash of that group's own sources (plus every header and host file)."""

import os
import shutil

import pytest

from kv_cache_quantization_05_amd import rocpd_summary as rs

CSRC = os.path.join(os.path.dirname(rs.__file__), "csrc")


@pytest.mark.parametrize("name,group,decode,prefill", [
    ("void tq::(anonymous namespace)::attend_mfma_kernel<3, 3, false, false>(tq::dev_tables, tq::dev_tables, tq::attend_args)",
     "attend_decode", True, False),
    ("void tq::v1::attend_merge_kernel<128>(tq::dev_tables, tq::attend_args)", "attend_decode", True, False),
    ("void tq::v1::attend_partial_kernel<128, 4, 4, false, 1>(tq::dev_tables, tq::dev_tables, tq::attend_args)",
     "attend_decode", True, False),
    ("void tq::v1::query_prep_kernel<128, false>(tq::dev_tables, float const*, float*, long)", "attend_decode", True, False),
    ("void tq::(anonymous namespace)::prefill32_kernel<128, 3, 3>(tq::dev_tables, tq::dev_tables, tq::prefill_args)",
     "attend_prefill", False, True),
    ("void tq::(anonymous namespace)::prefill_kernel<128, 3, 3, false, 2, 4>(tq::dev_tables, tq::dev_tables, tq::prefill_args)",
     "attend_prefill", False, True),
    ("void tq::(anonymous namespace)::rotate_back_kernel<128>(tq::dev_tables, float const*, float*)", "attend_prefill", False, True),
    ("void tq::v1::query_prep_kernel<128, false>(tq::dev_tables, float const*, float*, long)", "attend_prefill", False, True),
    ("void tq::v1::query_prep_kernel<256, true>(tq::dev_tables, float const*, float*, long)", "scores", False, False),
    ("void tq::(anonymous namespace)::scores_tile32_kernel<256, 4, true, true>(tq::dev_tables, tq::scores_args)", "scores", False, False),
    ("void tq::(anonymous namespace)::topk_merge_kernel(tq::scores_args)", "scores", False, False),
    ("void tq::(anonymous namespace)::encode_mfma_kernel<128, 3, false, true>(tq::dev_tables, tq::encode_args, tq::(anonymous namespace)::grid_index, unsigned int)",
     "encode", True, False),
    ("void tq::(anonymous namespace)::encode_qjl_mfma_kernel<128, 4, true>(tq::dev_tables, tq::encode_args, tq::(anonymous namespace)::grid_index, unsigned int)",
     "encode", True, False),
    ("__amd_rocclr_copyBuffer", None, True, False),
])
def test_kernels_fall_in_their_launch_groups(monkeypatch, name, group, decode, prefill):
    monkeypatch.setattr(rs, "_has_decode", [decode])
    monkeypatch.setattr(rs, "_has_prefill", [prefill])
    assert rs.group_of(name) == group


def test_every_hip_source_belongs_to_a_group():
    hips = {f for f in os.listdir(CSRC) if f.endswith(".hip")}
    owned = set().union(*rs.GROUP_SOURCES.values())
    # the no-allocation entry point's kernels are the decode kernels; its own
    # file holds only the host side of that call
    assert hips - owned <= {"tq_static.hip"}, hips - owned
    assert owned <= hips, owned - hips


def test_traffic_keys_follow_each_groups_sources(monkeypatch, tmp_path):
    pkg = tmp_path / "pkg"
    shutil.copytree(CSRC, pkg / "csrc")
    monkeypatch.setattr(rs, "PKG", str(pkg))
    before = {g: rs.kernel_source_hash(g) for g in rs.GROUP_SOURCES}
    # a change to a scorer source moves only the scorer's key
    with open(pkg / "csrc" / "tq_scores32.hip", "a") as f:
        f.write("\n// edit\n")
    after = {g: rs.kernel_source_hash(g) for g in rs.GROUP_SOURCES}
    assert after["scores"] != before["scores"]
    assert all(after[g] == before[g] for g in before if g != "scores")
    # a header change moves every key
    with open(pkg / "csrc" / "tq_device.h", "a") as f:
        f.write("\n// edit\n")
    again = {g: rs.kernel_source_hash(g) for g in rs.GROUP_SOURCES}
    assert all(again[g] != after[g] for g in after)
