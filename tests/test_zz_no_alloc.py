"""paged_decode_attn_kv8_noalloc (the decode with the library's fixed
scratch in place of a workspace) against paged_decode_attn_kv8 through the
C ABI: two calls in a row, the second on a smaller input, each bitwise equal
to the workspace entry's output for the same split size and kernel form and
within tolerance of the oracle; every output element written; a call
needing more than the fixed scratch is refused."""
import numpy as np
import pytest
import torch

from oracle import kv8_oracle as O
from paged_int8_kv_amd import binding as B
from paged_int8_kv_amd import workloads as W
from tests.kv8_testutil import (check_close, dev, gpu_decode, needs_gpu, oracle_cache, q_tensor,
                                upload_cache)

pytestmark = [pytest.mark.gpu, needs_gpu]


def noalloc_decode(case, cache, tps, form):
    qt = q_tensor(case)
    b, hq, d = qt.shape
    out = torch.full((b, hq, d), float("nan"), dtype=torch.float32, device=dev())
    B.paged_decode_attn_kv8_noalloc(
        qt, *cache, torch.from_numpy(case.block_table).to(dev()),
        torch.from_numpy(case.context_lens).to(dev()), int(case.context_lens.max()), out,
        tokens_per_split=tps, kernel_form=form)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("form", [B.DECODE_AUTO, B.DECODE_DOT, B.DECODE_MFMA,
                                  B.DECODE_MFMA_ONEPASS])
@pytest.mark.parametrize("tps", [0, 128])
def test_noalloc_matches_workspace_entry_two_calls(form, tps):
    big = W.llama8b_decode(batch=16)
    small = W.make_paged_case(batch=3, num_q_heads=32, num_kv_heads=8, head_dim=128,
                              context_lens=[700, 1, 2100], q_dtype="bf16", k_outliers=True,
                              seed=81)
    for case in (big, small):
        host = oracle_cache(case)
        cache = upload_cache(*host)
        got = noalloc_decode(case, cache, tps, form)
        want = gpu_decode(case, cache, tokens_per_split=tps, kernel_form=form)
        assert np.all(np.isfinite(got)), "an output element was not written"
        assert np.array_equal(got, want), f"noalloc != workspace entry, batch {case.batch}"
        ref = O.paged_decode(case.q, *host, case.block_table, case.context_lens)
        check_close(got, ref, f"noalloc batch {case.batch} form {form} tps {tps}")


def test_noalloc_refuses_beyond_scratch():
    case = W.make_paged_case(batch=2, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=[64, 64], seed=82)
    cache = upload_cache(*oracle_cache(case))
    qt = q_tensor(case)
    out = torch.zeros((2, 32, 128), dtype=torch.float32, device=dev())
    # a host bound of 1M tokens in 64-token splits of the one-pass form sizes
    # its partials beyond the scratch (the stream-K form's partials do not
    # grow with the context, so the form is named)
    with pytest.raises(B.Kv8Error) as e:
        B.paged_decode_attn_kv8_noalloc(
            qt, *cache, torch.from_numpy(case.block_table).to(dev()),
            torch.from_numpy(case.context_lens).to(dev()), 1 << 20, out, tokens_per_split=64,
            kernel_form=B.DECODE_MFMA_ONEPASS)
    assert e.value.status == B.KV8_ERR_WORKSPACE
