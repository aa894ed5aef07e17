"""The benchmark's closed-form work counts against the oracle's pair-by-pair
mask count (CPU only), so the reported TFLOP/s divide the right numerator."""
import numpy as np
import pytest

import bench
import swa_inputs as si
from oracle import oracle as orc


@pytest.mark.parametrize("name", list(si.PREFILL_WORKLOADS))
def test_useful_pairs_match_oracle_mask(name):
    c = si.PREFILL_WORKLOADS[name]()
    assert bench.useful_pairs(c) == orc.count_allowed(c.cu_seqlens, c.ids, c.window, c.mode)


def test_useful_flops_of_the_prefill_workloads():
    assert bench.useful_flops(si.prefill_4x1024_mha_d128()) == 34393292800
    assert bench.useful_flops(si.prefill_16k_gqa_d512()) == 1924212457472
    assert bench.useful_flops(si.prefill_vlm_4096_d256()) == 32208060416
    # 4 documents x 524,800 causal pairs (the window covers each document),
    # 16 heads, 4 * 320 flop per pair
    assert bench.useful_flops(si.prefill_4x1024_gqa_d320()) == 4 * 524800 * 16 * 4 * 320
    # the 16k window-4096 pair count of the D = 512 workload, 32 heads, D = 128
    assert bench.useful_flops(si.prefill_16k_mha_d128_w4k()) == 58722304 * 32 * 4 * 128


def test_decode_valid_rows():
    pos = np.array([0, 5, 3000, 40], np.int64)
    lo = np.array([0, 2, 0, 39], np.int64)
    np.testing.assert_array_equal(bench.decode_valid_rows(pos, lo, 1024), [1, 4, 1024, 2])


def test_every_workload_names_its_kernel():
    """bench.py --only accepts every named workload: each has the kernel and
    sources its roofline and traffic record refer to."""
    for name in list(si.PREFILL_WORKLOADS) + list(si.DECODE_WORKLOADS):
        assert name in bench.WORKLOAD_KERNELS, name
        bench.sources_hash(name)
