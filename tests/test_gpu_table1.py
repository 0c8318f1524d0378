"""Expert Coupling in MoE Pretraining, section II-B, Table I, through the library: on synthetic
correlated routing at 128 experts (top-2 and top-6) the GPU co-selection counts and the host
Algorithm 1 partition equal the oracle's, and the statistics the benchmark reports from the GPU
layout (dedup rows, tokens on one GPU) equal the oracle layout's, for EP 8/16/32 under both
placements; co-selection counts also at 256 and 512 experts. The statistics themselves are
reported beside the pages' rows by bench.py --table1."""
import numpy as np
import pytest
import torch

from dispatch_expert_gemm_amd import moe
from dispatch_expert_gemm_amd import workloads as WL
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


@pytest.mark.parametrize("E,k", [(128, 2), (128, 6), (256, 8), (512, 8)])
def test_coselect_counts_match_oracle(E, k):
    rng = np.random.default_rng(E + k)
    N = 4096
    idx = np.argsort(rng.random((N, E)) - (rng.random(E) < 0.1) * 0.5, axis=1)[:, :k]
    idx = idx.astype(np.int32)
    got = moe.moe_coselect_counts(torch.from_numpy(idx).to(DEV), E)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), O.coselect_counts(idx, E))


@pytest.mark.parametrize("k", [2, 6])
def test_table1_statistics_match_oracle(k):
    import bench
    c = WL.SHUFFLE_TRACES[bench.TABLE1_TRACES[k]]
    fit = WL.gen_shuffle_trace(c, "fit")[2][:16384]
    cur = WL.gen_shuffle_trace(c, "eval")[2]
    counts = moe.moe_coselect_counts(torch.from_numpy(fit).to(DEV), c.E).cpu().numpy()
    assert np.array_equal(counts, O.coselect_counts(fit, c.E))
    for P in (8, 16, 32):
        group, swaps = moe.moe_placement_partition(counts, P)
        want_group, want_swaps = O.partition(counts, P)
        assert np.array_equal(group, want_group) and swaps == want_swaps
        for pl in (None, group):
            lay = moe.Layout(c.T, c.E, k, P, 8)
            moe.moe_dispatch_layout(lay, torch.from_numpy(cur).to(DEV),
                                    None if pl is None else torch.from_numpy(pl).to(DEV))
            torch.cuda.synchronize()
            ref = O.layout(cur, O.contiguous_placement(c.E, P) if pl is None else pl, P)
            D = int(lay["pair_offsets"][P])
            assert D == ref["D"]
            got_tok = np.bincount(lay["pair_token"][:D].cpu().numpy(), minlength=c.T)
            want_tok = np.bincount(ref["pair_token"][:D], minlength=c.T)
            assert np.array_equal(got_tok, want_tok)
        print(f"[table1 top-{k} EP{P}] placement swaps {swaps}, contiguous and correlated "
              f"statistics equal the oracle's", flush=True)
