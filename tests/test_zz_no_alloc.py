"""paged_attn_decode_noalloc (the decode with its scratch in a fixed device
array, for callers that cannot allocate) against paged_attn_decode with a
caller workspace, through the C ABI: bit-identical outputs on two calls in a
row, the second on a smaller batch, and host-side rejection of a batch whose
scratch would exceed the array."""
import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_429_amd import binding as B
from synth import make_config_case
from tests.gpu_util import assert_close, dev_to_f64, np_to_dev, oracle_decode, upload_meta, upload_pools

pytestmark = pytest.mark.gpu


def _noalloc(c, q, kp, vp, tables, ctx, out):
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return B.lib().paged_attn_decode_noalloc(
        p(q), p(kp), p(vp), None, None, p(tables), c.max_blocks_per_seq, p(ctx), c.max_context_len, c.num_seqs,
        c.num_blocks, 16, c.n_heads, c.n_kv, c.d, B.PA_BF16, 16, p(out), 0, stream)


def test_noalloc_matches_workspace_decode(lib):
    """The 70B prefix-shared batch (prefix pass, split partials: about 51 MiB
    of scratch), then a smaller Llama-3-8B-shaped batch on the same array."""
    for c, seqs in ((make_config_case(3), [0, 31, 32, 200, 255]), (make_config_case(2, num_seqs=16), None)):
        kp, vp = upload_pools(c)
        tables, ctx = upload_meta(c)
        q = np_to_dev(c.q, "bf16")
        ref = B.decode(q, kp, vp, tables, ctx, n_kv_heads=c.n_kv, max_context_len=c.max_context_len)
        out = torch.full_like(q, float("nan"))
        assert _noalloc(c, q, kp, vp, tables, ctx, out) == 0
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), c.name
        got = dev_to_f64(out)
        want = oracle_decode(c, seqs=seqs)
        rows = list(range(c.num_seqs)) if seqs is None else seqs
        assert_close(got[rows], want[rows], "bf16", c.name)
        del kp, vp


def test_noalloc_rejects_batches_beyond_its_scratch(lib):
    """512 sequences of the prefix-shared shape need about 67 MiB: rejected
    with PA_ERR_SCRATCH before any device work (the output is untouched)."""
    c = make_config_case(2, num_seqs=4)
    kp, vp = upload_pools(c)
    tables, ctx = upload_meta(c)
    q = np_to_dev(c.q, "bf16")
    out = torch.full_like(q, 3.0)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = B.lib().paged_attn_decode_noalloc(p(q), p(kp), p(vp), None, None, p(tables), c.max_blocks_per_seq, p(ctx),
                                           4500, 512, c.num_blocks, 16, 64, 8, 128, B.PA_BF16, 16, p(out), 0, None)
    assert st == -7  # PA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
