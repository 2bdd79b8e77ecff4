"""The automatic choice among the decode kernel forms.  For shapes on each
side of the rule, a launch under KV8_DECODE_AUTO must be bitwise the launch
of the form the rule names:
- v_dot2 below 4 query heads per KV head;
- two-pass matrix-core from 4 heads per KV head for contexts of
  2049..8192 tokens in a grid bound of at most 1024 workgroups;
- stream-K matrix-core otherwise from 4 heads per KV head;
- INT4: one-pass matrix-core from 4 heads per KV head at d = 128, v_dot2 at
  d = 64.
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

FORMS = {"dot": B.DECODE_DOT, "mfma": B.DECODE_MFMA, "mfma1": B.DECODE_MFMA_ONEPASS,
         "sk": B.DECODE_STREAMK}


def run_forms(run):
    """run(kernel_form) under the automatic choice and every form."""
    return {name: run(which) for name, which in [("auto", B.DECODE_AUTO)] + list(FORMS.items())}


@pytest.mark.parametrize("hq,hkv,lens,expected", [
    (16, 8, [300, 700, 41], "dot"),              # G = 2
    (32, 8, [1500, 3000, 17, 999], "mfma"),      # G = 4, short contexts, small grid
    (32, 8, [9000, 100], "sk"),                  # G = 4, a context past 8192 tokens
    (32, 8, [2048, 700, 1], "sk"),               # G = 4, no context past 2048 tokens
    (32, 8, [4096] + [16] * 32, "sk"),           # G = 4, grid bound 33 * 4 * 8 > 1024
    (64, 8, [500, 2000, 1], "sk"),               # G = 8, no context past 2048 tokens
    (64, 8, [3000, 100, 2500], "mfma"),          # G = 8, mid-length contexts, small grid
    (64, 8, [9000, 700], "sk"),                  # G = 8, a context past 8192 tokens
])
def test_auto_form_int8(hq, hkv, lens, expected):
    case = W.make_paged_case(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                             context_lens=lens, q_dtype="bf16", k_outliers=True, seed=hq + sum(lens))
    kc, vc, ks, vs = oracle_cache(case)
    cache = upload_cache(kc, vc, ks, vs)
    outs = run_forms(lambda f: gpu_decode(case, cache, kernel_form=f))
    assert np.array_equal(outs["auto"], outs[expected]), f"auto is not {expected}"
    for other in FORMS:
        if other != expected:
            assert not np.array_equal(outs[expected], outs[other]), f"{expected} == {other}"
    ref = O.paged_decode(case.q, kc, vc, ks, vs, case.block_table, case.context_lens)
    check_close(outs["auto"], ref, f"auto form hq={hq} hkv={hkv}")


@pytest.mark.parametrize("lens,expected", [([1200, 77, 2500], "mfma1"), ([9000, 300], "mfma1")])
def test_auto_form_int4(lens, expected):
    """INT4 at d = 128 and G = 4 takes the one-pass matrix-core form, short
    or long contexts (the two-pass form is there on request)."""
    case = W.make_paged_case(batch=len(lens), num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=lens, q_dtype="bf16", k_outliers=True,
                             seed=91 + sum(lens))
    host = oracle_cache_int4(case)
    cache = upload_int4(*host)
    outs = run_forms(lambda f: gpu_decode_int4(case, cache, kernel_form=f))
    assert np.array_equal(outs["auto"], outs[expected])
    for other in FORMS:
        if other != expected:
            assert not np.array_equal(outs[expected], outs[other]), f"{expected} == {other}"
    ref = O.paged_decode_int4(case.q, *host, case.block_table, case.context_lens)
    check_close(outs["auto"], ref, "auto form int4")


def test_int4_head_dim_64_takes_dot():
    """The matrix-core forms serve INT4 at d = 128 only: at d = 64 every
    requested form runs the v_dot2 kernel."""
    case = W.make_paged_case(batch=2, num_q_heads=16, num_kv_heads=4, head_dim=64,
                             context_lens=[700, 33], q_dtype="bf16", seed=17)
    host = oracle_cache_int4(case)
    cache = upload_int4(*host)
    outs = run_forms(lambda f: gpu_decode_int4(case, cache, kernel_form=f))
    for name in ("auto", "mfma", "mfma1", "sk"):
        assert np.array_equal(outs[name], outs["dot"]), name
