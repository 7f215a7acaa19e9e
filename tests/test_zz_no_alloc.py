"""lrkv_decode_noalloc against lrkv_decode, through the C ABI: two calls in a row on the
same fixed scratch, the second with a smaller input; each output must equal lrkv_decode's
bit for bit (the same kernels and split) and be within the bar of the float64 oracle."""

import numpy as np
import pytest
import torch

import factored_rank_kv_amd as F
import oracle as O
from lrkv_case import from_dev, iid_case, layout_c, log, max_rel_err, tolerance

pytestmark = pytest.mark.gpu


def run_noalloc(case, chunk_tokens=0):
    d = case.dev
    out = torch.full(case.q_codes.shape, -1, dtype=d["q"].dtype, device="cuda:0")
    F.lrkv_decode_noalloc(layout_c(case.L), d["q"], case.B, case.q_len, d["BK"], d["BV"],
                          d["pool"], d["table"], case.table.shape[1], d["lens"],
                          int(case.lens.max()), chunk_tokens, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_decode_two_calls(order):
    big = iid_case(301, 16, 128, 56, O.BF16, [4096] * 8, permute=False)  # 8 x 4096 tokens
    small = iid_case(302, 16, 128, 56, O.BF16, [5, 300, 17], permute=True, fill=0x7FC0)
    for what, case in (("B=8 x 4096", big), ("B=3 ragged", small)):
        log(f"no-alloc decode, {what}")
        got = run_noalloc(case)
        want = case.run()
        assert torch.equal(got.cpu(), want.cpu()), what
        err = max_rel_err(from_dev(got, O.BF16), case.reference())
        log(f"no-alloc {what}: bit-identical to lrkv_decode, max rel err {err:.3e}")
        assert err <= tolerance(O.BF16)


def test_noalloc_balanced_then_chunked_other_shape():
    """The balanced split (16+ requests) at the 32-head shape, then a smaller chunked call."""
    lens = [0, 1, 17, 300, 48, 1000, 33, 16] * 3
    a = iid_case(303, 32, 128, 32, O.BF16, lens, permute=True, fill=0x7FC0)
    b = iid_case(304, 32, 128, 32, O.BF16, [64, 129], permute=True, fill=0x7FC0)
    for what, case in (("balanced B=24", a), ("chunked B=2", b)):
        got = run_noalloc(case)
        want = case.run()
        assert torch.equal(got.cpu(), want.cpu()), what
        live = case.lens > 0
        err = max_rel_err(from_dev(got, O.BF16)[live], case.reference()[live])
        log(f"no-alloc {what}: bit-identical to lrkv_decode, max rel err {err:.3e}")
        assert err <= tolerance(O.BF16)


def test_noalloc_rejects_calls_beyond_its_scratch():
    case = iid_case(305, 16, 128, 56, O.BF16, [4096] * 8, permute=False)
    d = case.dev
    out = torch.empty(case.q_codes.shape, dtype=d["q"].dtype, device="cuda:0")
    # 16-token chunks: 256 chunks x 8 requests x 16 heads x 752 B = 24 MiB of partials
    st = F.lrkv_decode_noalloc(layout_c(case.L), d["q"], 8, 1, d["BK"], d["BV"], d["pool"],
                               d["table"], case.table.shape[1], d["lens"], 4096, 16, out,
                               check=False)
    assert st == F.LRKV_ERR_SCRATCH
