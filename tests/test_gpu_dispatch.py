"""The automatic choice among the decode kernel forms.  For shapes on each
side of the rule, a launch under KV8_DECODE_AUTO must be bitwise the launch
of the form the rule names:
- v_dot2 below 4 query heads per KV head;
- two-pass matrix-core at 4 for short contexts in a small grid;
- one-pass matrix-core for long contexts, from 8 heads per KV head, and for
  INT4 at d = 128.
The named form must also differ from the other forms on that input, so that
the comparison can tell them apart.  Each result is checked against the
oracle too."""
import numpy as np
import pytest

from oracle import kv8_oracle as O
from paged_int8_kv_amd import binding as B
from paged_int8_kv_amd import workloads as W
from tests.kv8_testutil import check_close, gpu_decode, needs_gpu, oracle_cache, upload_cache
from tests.test_gpu_int4kv import gpu_decode_int4, oracle_cache_int4, upload_int4

pytestmark = [pytest.mark.gpu, needs_gpu]

FORMS = {"dot": B.DECODE_DOT, "mfma": B.DECODE_MFMA, "mfma1": B.DECODE_MFMA_ONEPASS}


def run_forms(run):
    outs = {}
    try:
        for name, which in [("auto", B.DECODE_AUTO)] + list(FORMS.items()):
            B.kv8_set_decode_kernel(which)
            outs[name] = run()
    finally:
        B.kv8_set_decode_kernel(B.DECODE_AUTO)
    return outs


@pytest.mark.parametrize("hq,hkv,lens,expected", [
    (16, 8, [300, 700, 41], "dot"),              # G = 2
    (32, 8, [1500, 3000, 17, 999], "mfma"),      # G = 4, short contexts, small grid
    (32, 8, [9000, 100], "mfma1"),               # G = 4, a context past 8192 tokens
    (64, 8, [500, 2000, 1], "mfma1"),            # G = 8
])
def test_auto_form_int8(hq, hkv, lens, expected):
    case = W.make_paged_case(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                             context_lens=lens, q_dtype="bf16", k_outliers=True, seed=hq + sum(lens))
    kc, vc, ks, vs = oracle_cache(case)
    cache = upload_cache(kc, vc, ks, vs)
    outs = run_forms(lambda: gpu_decode(case, cache))
    assert np.array_equal(outs["auto"], outs[expected]), f"auto is not {expected}"
    for other in FORMS:
        if other != expected:
            assert not np.array_equal(outs[expected], outs[other]), f"{expected} == {other}"
    ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    check_close(outs["auto"], ref, f"auto form hq={hq} hkv={hkv}")


def test_auto_form_int4():
    """INT4 has two forms: one-pass matrix-core at d = 128 from G = 4, else
    v_dot2 (the two-pass setting falls back to v_dot2)."""
    case = W.make_paged_case(batch=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=[1200, 77, 2500], q_dtype="bf16", k_outliers=True,
                             seed=91)
    host = oracle_cache_int4(case)
    cache = upload_int4(*host)
    outs = run_forms(lambda: gpu_decode_int4(case, cache))
    assert np.array_equal(outs["auto"], outs["mfma1"])
    assert np.array_equal(outs["mfma"], outs["dot"])
    assert not np.array_equal(outs["mfma1"], outs["dot"])
    ref = O.paged_decode_int4(case.q, *host, case.block_table, case.context_lens)
    check_close(outs["auto"], ref, "auto form int4")
