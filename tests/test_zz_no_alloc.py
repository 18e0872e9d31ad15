"""The allocation-free permutation (moe_permute_noalloc) against moe_permute, through the C ABI:
bit-exact sorted_pairs[:n_loc], group_offsets and pair_pos on two calls in a row, the second with a
smaller input (the library's scratch array then holds the first call's counts), and on an input
small enough to need no scratch at all."""
import numpy as np
import pytest
import torch

from expert_grouped_gemm_softmax_amd import ops
from expert_grouped_gemm_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu


def _blob(T, E, k, seed):
    # routing blob of the workloads' recipe (seeded fp32 logits), routed by the library
    cfg = W.MoEConfig("noalloc", T=T, H=64, E=E, k=k, I=64, e_first=0, e_local=1, seed=seed)
    logits = torch.from_numpy(W.make_inputs(cfg)["logits"]).to("cuda:0")
    _, _, blob = ops.route_packed(logits, k, write_ids=False)
    return blob


def _check(blob, e_first, e_local):
    _, T, k = blob.shape
    dev = blob.device
    ref_sp, ref_off, ref_pp = ops.permute(blob, e_first, e_local)
    sp = torch.full((T * k,), -5, dtype=torch.int32, device=dev)
    off = torch.full((e_local + 1,), -5, dtype=torch.int32, device=dev)
    pp = torch.full((T * k,), -5, dtype=torch.int32, device=dev)
    ops.permute_noalloc(blob, e_first, e_local, sp, off, pp)
    torch.cuda.synchronize()
    n = int(ref_off[-1])
    assert torch.equal(off, ref_off)
    assert torch.equal(sp[:n], ref_sp[:n])
    assert torch.equal(pp, ref_pp)
    assert torch.all(sp[n:] == -5)                      # rows past n_loc are left untouched
    return n


def test_permute_noalloc_matches_permute_on_two_calls_in_a_row():
    n1 = _check(_blob(8192, 512, 10, seed=3), 0, 64)         # 81920 pairs: 160 chunks of counts
    n2 = _check(_blob(3000, 96, 8, seed=4), 16, 40)          # smaller: 47 chunks, fewer experts
    n3 = _check(_blob(700, 64, 6, seed=5), 8, 24)            # 4200 pairs: no scratch needed
    assert n1 > n2 > n3 > 0
    print("n_loc", n1, n2, n3)


def test_permute_noalloc_near_its_scratch_limit():
    # 1024 local experts and 1024 chunks of 512 pairs: the counts fill the whole array
    blob = _blob(1024 * 512 // 64, 1024, 64, seed=6)
    n = _check(blob, 0, 1024)
    assert n == 1024 * 512
