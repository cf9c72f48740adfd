"""attn_decode_paged_noalloc: the paged decode with the library's own scratch
array instead of a caller workspace.  Through the C ABI, its output must equal
attn_decode_paged's bit for bit (the same kernels run on the same schedule),
on two calls in a row, the second with a smaller input; sizes whose workspace
exceeds the scratch array are refused before anything runs.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from exact_softmax_attention_amd import _lib, attn_decode_paged

pytestmark = pytest.mark.gpu

ATTN_E_WORKSPACE = -5


def _call_noalloc(d, scale, window=0):
    q, kc = d["q"], d["kcache"]
    B, Hq, hd = q.shape
    num_blocks, block_size, Hkv, _ = kc.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    code = _lib.lib().attn_decode_paged_noalloc(
        q.data_ptr(), kc.data_ptr(), d["vcache"].data_ptr(), d["block_table"].data_ptr(),
        d["seq_lens"].data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, hd, block_size,
        d["block_table"].shape[1], num_blocks, window, scale,
        torch.cuda.current_stream().cuda_stream)
    return code, out, lse


def _compare(d, scale, window, what):
    print(f"no-alloc decode: {what}", flush=True)
    code, out, lse = _call_noalloc(d, scale, window)
    assert code == 0, _lib.status_str(code)
    ref_o, ref_l = attn_decode_paged(d["q"], d["kcache"], d["vcache"], d["block_table"],
                                     d["seq_lens"], scale=scale, window=window)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o), what
    assert torch.equal(lse, ref_l), what


def test_noalloc_decode_equals_workspace_decode_twice():
    # the paged decode workload first (16 sequences of 8000..32000 tokens)
    pc = workloads.PAGED_CONFIGS["paged_decode_16x32k"]
    big = {k: v.cuda() for k, v in workloads.make_paged_config(pc).items()}
    _compare(big, pc.scale, 0, "paged_decode_16x32k")
    del big
    # then a smaller batch: other head counts, head dim 64, a window, an empty sequence
    lens = [0, 700, 37]
    small = workloads.make_paged(3, 8, 2, 64, 16, 200, 60, 7301, seq_lens=lens)
    small = {k: v.cuda() for k, v in small.items()}
    _compare(small, float(np.float32(1.0 / math.sqrt(64))), 100, "3 sequences, 8x2 heads, d 64")


def test_noalloc_refuses_sizes_beyond_the_scratch():
    # 64 query heads of 128: the partials need more than the 16 MiB array
    q = torch.zeros((1, 64, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones((1,), dtype=torch.int32, device="cuda")
    d = {"q": q, "kcache": kc, "vcache": kc, "block_table": table, "seq_lens": lens}
    code, _, _ = _call_noalloc(d, 0.088)
    assert code == ATTN_E_WORKSPACE
