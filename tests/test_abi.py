"""The C-ABI library loads, exports every declared symbol, validates its
arguments before any launch, and its host-only subsample draw matches the
oracle bit for bit.  CPU only: no call here reaches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import group_sparse_swiglu_amd as E
from oracle import esg_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "esg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(esg_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = E.lib()
    declared = _declared_functions()
    assert len(declared) >= 13
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(E.EXPORTED_SYMBOLS) == declared


def test_status_strings():
    lib = E.lib()
    for code in range(5):
        assert lib.esg_status_string(code)
    assert lib.esg_version() >= 10000


@pytest.mark.parametrize("d_ff,gs,spg,seed", [(2048, 64, 8, 0), (2688, 128, 16, 0), (5504, 128, 16, 0),
                                              (512, 32, 32, 0), (96, 16, 5, 77), (16384, 16, 3, 2**63 + 5)])
def test_subsample_matches_oracle(d_ff, gs, spg, seed):
    sub, got_spg = E.make_subsample_index(d_ff, gs, spg, seed)
    assert got_spg == spg
    assert np.array_equal(sub.numpy(), O.make_subsample_index(d_ff, gs, spg, seed))


@pytest.mark.parametrize("args", [(100, 32, 8), (128, 12, 8), (128, 32, 33), (128, 32, 0), (32, 32, 4),
                                  (128, 8, 4)])
def test_subsample_shape_rules(args):
    with pytest.raises(E.EsgError):
        E.make_subsample_index(*args, 0)


def _sizes(*args):
    sv, fw, bw = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = E.lib().esg_sparse_swiglu_workspace_size(*args, ctypes.byref(sv), ctypes.byref(fw), ctypes.byref(bw))
    return st, sv.value, fw.value, bw.value


def test_workspace_sizes_and_shape_rules():
    st, sv, fw, bw = _sizes(8192, 768, 2048, 64, 8, E.ESG_BF16, 0)
    assert st == 0 and sv > 0 and fw > 8192 * 8 * 768 * 2 and bw > fw
    # shape rules of the README's parameter table
    assert _sizes(8192, 760, 2048, 64, 8, E.ESG_BF16, 0)[0] == 2       # d_model % 16
    assert _sizes(8192, 768, 2048, 48, 8, E.ESG_BF16, 0)[0] == 2       # gs not a power of two
    assert _sizes(8192, 768, 2048, 8, 8, E.ESG_BF16, 0)[0] == 2        # gs < 16
    assert _sizes(8192, 768, 64, 64, 1, E.ESG_BF16, 0)[0] == 2         # fewer than two groups
    assert _sizes(8192, 768, 2048, 64, 33, E.ESG_BF16, 0)[0] == 2      # k > G
    assert _sizes(8192, 768, 2048, 64, 8, 7, 0)[0] == 2                # dtype
    assert _sizes(2**28, 768, 2048, 64, 8, E.ESG_BF16, 0)[0] == 2      # tokens*k >= 2^31
    assert _sizes(-1, 768, 2048, 64, 8, E.ESG_BF16, 0)[0] == 1
    # dense limit (idx = NULL): nothing saved, no forward scratch, a chunked backward workspace
    st, sv, fw, bw = _sizes(65536, 2048, 5504, 128, 43, E.ESG_BF16, 1)
    assert st == 0 and sv == 0 and fw == 0 and bw >= 3 * 43 * 128 * 8192 * 2
    assert _sizes(65536, 2048, 5504, 128, 42, E.ESG_BF16, 1)[0] == 1   # dense needs k == G
    assert _sizes(256, 128, 512, 32, 16, E.ESG_F32, 1)[0] == 2         # dense kernels are bf16
    assert _sizes(256, 2064, 512, 32, 16, E.ESG_BF16, 1)[0] == 2       # d_model above 2048


def test_forward_scratch_holds_split_partials_exactly_under_the_tile_limit():
    # 16 groups of 64, k = 2, d = 80: tiles are bounded by floor((T*k + 16*127)/128),
    # 128 at 7239 tokens (two-launch forward: fp32 [hg; hu] of up to 4 K ranges,
    # 4 * 128 * 128 * 4 bytes per tile) and 129 at 7240 (one launch, no such
    # buffer), so the scratch shrinks across the limit by about 32 MB.
    st0, _, fw_split, _ = _sizes(7239, 80, 1024, 64, 2, E.ESG_BF16, 0)
    st1, _, fw_one, _ = _sizes(7240, 80, 1024, 64, 2, E.ESG_BF16, 0)
    assert st0 == 0 and st1 == 0
    partial_bytes = 128 * 4 * 128 * 128 * 4
    assert partial_bytes - 4096 <= fw_split - fw_one + 128 * 80 * 2 <= partial_bytes + 4096
    # one tile below the limit both sizes hold the buffer
    assert _sizes(7238, 80, 1024, 64, 2, E.ESG_BF16, 0)[2] <= fw_split
    # fp32 launches never split
    _, _, f32_a, _ = _sizes(7239, 80, 1024, 64, 2, E.ESG_F32, 0)
    _, _, f32_b, _ = _sizes(7240, 80, 1024, 64, 2, E.ESG_F32, 0)
    assert f32_a <= f32_b < f32_a + 64 * 1024


def _saved_rows(T, d, F, gs, k):
    """Bucket rows implied by the size of `saved`: per row 4 bytes of ptoken,
    2 * gs bytes each of bf16 hg and hu, and 4 bytes of tile group per 128
    rows; besides them T*k*4 bytes of pinv and the group offsets."""
    _, sv, _, _ = _sizes(T, d, F, gs, k, E.ESG_BF16, 0)
    return (sv - T * k * 4) / (4 + 4 / 128 + 2 * 2 * gs)


@pytest.mark.parametrize("T,d,F,gs,k,pad", [(32768, 2048, 5504, 128, 11, 256), (23335, 2048, 5504, 128, 11, 256),
                                            (23334, 2048, 5504, 128, 11, 128), (16384, 1024, 2688, 128, 5, 128),
                                            (8192, 768, 2048, 64, 8, 128), (100, 2048, 5504, 128, 11, 128)])
def test_training_layout_pads_each_group_to_its_tile_unit(T, d, F, gs, k, pad):
    """Each group's bucket holds at most n_g + pad - 1 rows, rounded to whole
    pads of 128-position tiles: pairs of tiles (pad 256) where the forward and
    the dh + dx kernels take two tiles of one group (bf16, 128-neuron blocks,
    at least 2048 single tiles by the bound floor((T*k + G*127)/128): 23335
    tokens at the 1.3B shape, not 23334), single tiles otherwise (64-neuron
    blocks; 128-neuron launches under 2048 tiles, e.g. the 370M shape; under
    128 tiles 128-neuron groups take 64-neuron blocks)."""
    G = F // gs
    per = pad // 128
    tiles = (T * k + G * (pad - 1)) // 128
    tiles = (tiles + per - 1) // per * per
    rows = _saved_rows(T, d, F, gs, k)
    assert abs(rows - tiles * 128) < 16, (rows, tiles * 128)


def test_entry_points_reject_bad_arguments_before_launch():
    lib = E.lib()
    # NULL weights / misaligned pointers / bad shapes return before any HIP call
    assert lib.esg_grouped_topk_select(None, None, 1, 16, 64, 128, 32, 2, None, 0, None, None, None, None) == 1
    assert lib.esg_grouped_topk_select(8, 32, 1, 16, 64, 128, 32, 2, None, 0, None, 64, None, None) == 1
    assert lib.esg_grouped_topk_select(32, 32, 1, 16, 64, 128, 32, 5, None, 0, None, 64, None, None) == 2
    assert lib.esg_grouped_topk_select(32, 32, 1, 16, 64, 128, 32, 2, 64, 40, None, 64, None, None) == 2
    # the workspace variant: same checks, plus a misaligned workspace
    assert lib.esg_grouped_topk_select_ws(None, None, 1, 16, 64, 128, 32, 2, None, 0, None, None, None, None, 0,
                                          None) == 1
    assert lib.esg_grouped_topk_select_ws(32, 32, 1, 16, 64, 128, 32, 2, None, 0, None, 64, None, 8, 4096,
                                          None) == 1
    assert lib.esg_grouped_topk_select_ws(32, 32, 1, 16, 64, 128, 32, 5, None, 0, None, 64, None, 64, 4096,
                                          None) == 2
    need = ctypes.c_size_t()
    assert lib.esg_grouped_topk_select_workspace_size(64, 5504, 128, ctypes.byref(need)) == 0
    assert need.value == 64 * 43 * 4                      # an fp32 [tokens, G] energy table
    assert lib.esg_grouped_topk_select_workspace_size(64, 5504, 100, ctypes.byref(need)) == 1
    assert E.select_workspace_size(0, 2048, 64) == 0
    assert lib.esg_sparse_swiglu_fwd(32, 32, 32, 32, 1, 16, 64, 128, 32, 2, 64, 64, 64, 0, 64, 0, None, None) == 3
    assert lib.esg_sparse_swiglu_fwd(32, None, 32, 32, 1, 16, 64, 128, 32, 2, 64, 64, 64, 1 << 30, 64, 1 << 30,
                                     None, None) == 1
    assert lib.esg_sparse_swiglu_bwd(32, 32, 32, 32, 32, 1, 16, 64, 128, 32, 2, 64, 64, 0, 64, 64, 64, 64, 64, 0,
                                     None) == 3
    # dense (idx NULL): k must equal G; fp32 dense is not provided
    assert lib.esg_sparse_swiglu_fwd(32, 32, 32, 32, 1, 16, 64, 128, 32, 2, None, 64, None, 0, None, 0, None,
                                     None) == 1
    assert lib.esg_sparse_swiglu_fwd(32, 32, 32, 32, 0, 16, 64, 128, 32, 4, None, 64, None, 0, None, 0, None,
                                     None) == 2
    assert lib.esg_sparse_swiglu_bwd(32, 32, 32, 32, 32, 1, 16, 64, 128, 32, 4, None, None, 0, 64, 64, 64, 64, 64,
                                     16, None) == 3   # dense backward scratch too small
    assert lib.esg_update_load_balance_bias(None, 64, 64, 0.25, 1e-3, 0.5, 0.99, 4, None) == 1
    assert lib.esg_update_load_balance_bias_from_counts(64, 64, 64, 0, 0.25, 1e-3, 0.5, 0.99, 4, None) == 1
    # bias update from a saved routing: NULL saved, bad shape, saved too small
    assert lib.esg_update_load_balance_bias_from_routing(64, 64, None, 1 << 20, 64, 64, 256, 32, 2, 1, 0.25, 1e-3,
                                                         0.5, 0.99, None) == 1
    assert lib.esg_update_load_balance_bias_from_routing(64, 64, 64, 1 << 20, 64, 60, 256, 32, 2, 1, 0.25, 1e-3,
                                                         0.5, 0.99, None) == 2
    assert lib.esg_update_load_balance_bias_from_routing(64, 64, 64, 16, 64, 64, 256, 32, 2, 1, 0.25, 1e-3, 0.5,
                                                         0.99, None) == 3
    need = ctypes.c_size_t()
    assert lib.esg_bucket_workspace_size(100, 200, 300, ctypes.byref(need)) == 2   # k above the bucket limit
    assert lib.esg_bucket_workspace_size(100, 4, 2000, ctypes.byref(need)) == 2   # G above 1024
    assert lib.esg_bucket_workspace_size(100, 4, 16, ctypes.byref(need)) == 0 and need.value > 0
    assert lib.esg_bucket_by_group(64, 100, 4, 16, 64, 64, 64, None, 64, 0, None) == 3


def test_timing_api_without_launches():
    E.timing_reset()
    E.timing_enable(True)
    assert E.timing_read("fwd_grouped") == (0.0, 0)
    E.timing_enable(False)


def test_sigmoid_topk_argument_checks():
    lib = E.lib()
    assert lib.esg_sigmoid_topk_supported(256, 8) == 1
    assert lib.esg_sigmoid_topk_supported(2048, 32) == 1
    assert lib.esg_sigmoid_topk_supported(43, 11) == 1
    for e, k in ((2049, 8), (8, 33), (4, 5), (4, 0), (0, 1)):
        assert lib.esg_sigmoid_topk_supported(e, k) == 0
    null = None
    # tokens == 0 enqueues nothing and needs no buffers
    assert lib.esg_sigmoid_topk_routing(null, null, 1, 0, 256, 8, 1.0, 0, null, null, null) == 0
    assert lib.esg_sigmoid_topk_routing(null, null, 1, -1, 256, 8, 1.0, 0, null, null, null) == 1
    assert lib.esg_sigmoid_topk_routing(null, null, 0, 4, 256, 8, 1.0, 0, null, null, null) == 1
    assert lib.esg_sigmoid_topk_routing(null, null, 1, 4, 256, 40, 1.0, 0, null, null, null) == 2
    assert lib.esg_sigmoid_topk_routing(null, null, 1, 4, 256, 8, 1.0, 0, null, null, null) == 1


def test_leaky_mlp_sizes_and_argument_checks():
    lib = E.lib()
    sv, sc = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.esg_leaky_mlp_workspace_size(0, 512, 1792, ctypes.byref(sv), ctypes.byref(sc)) == 0
    assert sv.value == 0
    assert lib.esg_leaky_mlp_workspace_size(1000, 136, 456, ctypes.byref(sv), ctypes.byref(sc)) == 0
    assert sv.value >= 2 * 1000 * 456 * 2 and sc.value >= 1000 * 456 * 2
    assert lib.esg_leaky_mlp_workspace_size(10, 100, 64, ctypes.byref(sv), ctypes.byref(sc)) == 2   # d % 8
    assert lib.esg_leaky_mlp_workspace_size(-1, 64, 64, ctypes.byref(sv), ctypes.byref(sc)) == 1
    assert lib.esg_leaky_mlp_workspace_size(2 ** 20, 2048, 2048, ctypes.byref(sv), ctypes.byref(sc)) == 2
    null = None
    assert lib.esg_leaky_mlp_fwd(null, null, null, 0, 64, 64, null, null, 0, null) == 0
    assert lib.esg_leaky_mlp_fwd(null, null, null, 4, 64, 64, null, null, 0, null) == 1
