"""The backward's work order (GPU): the Delta phase writes, for the dK/dV and
the dQ kernels, the order in which they take their blocks (128 keys for
dK/dV; 128 or 256 queries for dQ, by the block-height rule below). Each list
must be a permutation of the blocks (or some block would be computed twice and
another never), sorted by cost, heaviest first, ties by block index.

A block's cost is the number of 64-row tiles of the other operand that the
mask lets it see: under a causal mask key j sees queries j.. of its segment and
query i sees keys up to i; with packing only its own segment; otherwise the
whole sequence.
"""
import os

import numpy as np
import pytest

import seeded_inputs as si
from tests.gpu_helpers import dev_i32

pytestmark = pytest.mark.gpu


def _segment(cu, i):
    s = int(np.searchsorted(cu, i, side="right")) - 1
    return int(cu[s]), int(cu[s + 1])


def _split(B, Hq, Hkv, S):
    units = B * Hkv * (-(-S // 128))
    return 1 if units >= 1024 else min(Hq // Hkv, -(-1024 // units))


def _ksplit(B, Hq, S):
    units = B * Hq * (-(-S // 128))
    return 1 if units >= 1024 else min(4, -(-1024 // units))


def _dq_rows(S, D, causal, packed, nk):
    """Rows of a dQ block: 256 (8 waves) for D = 128 without packing or key
    split from S = 16384 causal / 4096 non-causal, else 128; ATTN_DQ_WAVES=4|8
    forces it unless the key tiles are split."""
    if nk > 1:
        return 128
    forced = os.environ.get("ATTN_DQ_WAVES", "")
    if forced in ("4", "8"):
        return 32 * int(forced)
    if packed or D != 128:
        return 128
    return 256 if S >= (16384 if causal else 4096) else 128


def _cost(cu, S, causal, pass_, blk, rows=128):
    first, last = blk * rows, min(blk * rows + rows, S) - 1
    if pass_ == 0:  # keys first..last: the union of the queries they see
        lo = first if causal else _segment(cu, first)[0]
        hi = _segment(cu, last)[1]
    else:  # queries first..last: the union of the keys they see
        lo = _segment(cu, first)[0]
        hi = last + 1 if causal else _segment(cu, last)[1]
    return -(-hi // 64) - lo // 64


CASES = [
    (65, True, None),
    (300, False, None),
    (1000, True, [200, 13, 300, 487]),
    (4096, True, None),
    (32768, True, si.packed_lengths(np.random.default_rng(4))),
    (32768, False, si.packed_lengths(np.random.default_rng(7))),
    (20000, False, None),
    (70000, True, None),
]


@pytest.mark.parametrize("S,causal,lengths", CASES)
def test_block_order(S, causal, lengths):
    import torch
    import long_context_exact_fwd_amd as lca
    print(f"order S={S} causal={causal} lengths={lengths}", flush=True)
    B, Hq, Hkv, D = 1, 8, 1, 128
    z = torch.zeros((B, S, Hq, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, Hq, S), dtype=torch.float32, device="cuda")
    cu_h = si.cu_seqlens_from_lengths(lengths) if lengths else np.array([0, S], dtype=np.int32)
    cu = dev_i32(cu_h) if lengths else None
    nbytes = lca.bwd_workspace_bytes(B, Hq, Hkv, S, D)
    ws = torch.full((nbytes // 4,), -7, dtype=torch.int32, device="cuda")
    lca.bwd(z, kv, kv, z, lse, z, causal=causal, cu_seqlens=cu, workspace=ws, phases=lca.BWD_DELTA)
    torch.cuda.synchronize()
    nblk = -(-S // 128)
    ns, nk = _split(B, Hq, Hkv, S), _ksplit(B, Hq, S)
    rows = _dq_rows(S, D, causal, lengths is not None, nk)
    nqblk = -(-S // rows)
    G = Hq // Hkv
    off = 2 * B * Hq * (-(-S // 64) * 64)  # int32 words before the order
    order = ws[off:off + nblk * ns + nqblk * nk].cpu().numpy()
    # dK/dV entries e = key block * ns + share of the group's heads; cost = tiles * heads in the share.
    # dQ entries e = query block * nk + share of the block's key tiles; cost = tiles in the share.
    share = lambda n, m, i: (i + 1) * n // m - i * n // m
    for pass_, got, n in ((0, order[:nblk * ns], nblk * ns), (1, order[nblk * ns:], nqblk * nk)):
        assert sorted(got.tolist()) == list(range(n)), f"pass {pass_}: not a permutation"
        if pass_ == 0:
            keys = [(-_cost(cu_h, S, causal, 0, int(e) // ns) * share(G, ns, int(e) % ns), int(e)) for e in got]
        else:
            keys = [(-share(_cost(cu_h, S, causal, 1, int(e) // nk, rows), nk, int(e) % nk), int(e)) for e in got]
        assert keys == sorted(keys), f"pass {pass_}: not heaviest first"
