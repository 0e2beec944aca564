"""The GPU tests' all-token combine checker on the CPU: it accepts the
oracle's own result (rounded to float32 / bf16) and catches one element off."""

import numpy as np
import pytest

import oracle
from workloads import gen

from gpu_util import check_combine_all


@pytest.mark.parametrize("out_f32", [True, False])
def test_chunked_checker_accepts_the_oracle_and_catches_one_element(out_f32):
    b = gen.make_batch(gen.custom(5000, 64, 16, 4, 4, seed=3))
    p = oracle.route_plan(b.topk_idx, 16, 4)
    recv = oracle.dispatch(b.x, p)
    ref = oracle.combine(recv, b.topk_w, p)
    out = ref.astype(np.float32) if out_f32 else oracle.f32_to_bf16_rne(ref.astype(np.float32))
    check_combine_all(out, recv, b.topk_w, p["slot_of"], out_f32, "oracle")
    bad = out.copy()
    if out_f32:
        bad[4321, 7] = bad[4321, 7] * 1.01 + 0.01
    else:
        bad[4321, 7] = bad[4321, 7] + np.uint16(2)   # two bf16 ulps
    with pytest.raises(AssertionError, match="tokens 4096..4999"):
        check_combine_all(bad, recv, b.topk_w, p["slot_of"], out_f32, "planted")
