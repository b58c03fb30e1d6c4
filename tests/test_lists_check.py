"""CPU tests of the host-side list checker and of the binding's shape checks.

The attention kernels read q_idx / key_idx without bounds checks, so a bad
list must be caught before a launch: by cluster_attn_check_lists (values)
and by the Python binding (shapes).  Nothing here touches a GPU.
"""

import numpy as np
import pytest
import torch

import gathered_local_attention_amd as ca
import oracle as O
from gen import make_case


@pytest.fixture(scope="module")
def lists():
    case = make_case("stage1", B=2, tensors=False)
    perm, _, key = O.build_neighbors(case["coords"], case["cfg"].G)
    return torch.from_numpy(perm.reshape(2, -1, 8).copy()), torch.from_numpy(key.copy()), 2048


def test_valid_lists_pass(lists):
    q_idx, key_idx, N = lists
    ca.check_lists(q_idx, key_idx, N)
    ca.check_lists(q_idx.reshape(2, -1), key_idx, N)     # flat q_idx form
    k2 = key_idx.clone()
    k2[0, 3, 40:] = -1                                    # -1 slots are allowed
    ca.check_lists(q_idx, k2, N)


@pytest.mark.parametrize("where,value,msg", [
    ("key", 2048, "outside"),      # one past the end
    ("key", -2, "outside"),
    ("q", 5000, "outside"),
    ("q0", -1, "member 0"),
    ("dup", None, "twice"),
])
def test_bad_values_are_named(lists, where, value, msg):
    q_idx, key_idx, N = lists
    q, k = q_idx.clone(), key_idx.clone()
    if where == "key":
        k[1, 17, 9] = value
    elif where == "q":
        q[1, 3, 2] = value
    elif where == "q0":
        q[0, 7, 0] = value
    else:
        q[0, 9, 1] = q[0, 9, 2]
    with pytest.raises(ca.ClusterAttnError, match=msg):
        ca.check_lists(q, k, N)


def test_partial_clusters_and_packed_batch():
    # 13 tokens: one full cluster and a partial one of 5 members, then -1s
    q = torch.tensor([[[0, 1, 2, 3, 4, 5, 6, 7], [8, 9, 10, 11, 12, -1, -1, -1]]], dtype=torch.int32)
    k = torch.randint(0, 13, (1, 2, 48), dtype=torch.int32)
    ca.check_lists(q, k, 13)
    bad = q.clone()
    bad[0, 1, 6] = 12                                     # a token after a -1 (and twice)
    with pytest.raises(ca.ClusterAttnError):
        ca.check_lists(bad, k, 13)
    missing = q.clone()
    missing[0, 1, 4] = -1                                 # token 12 in no cluster
    with pytest.raises(ca.ClusterAttnError, match="holds 12 of the 13"):
        ca.check_lists(missing, k, 13)
    # packed batch: [Ct, cs] / [Ct, nk] with global ids, images of 13 and 3 tokens
    qp = torch.tensor([[0, 1, 2, 3, 4, 5, 6, 7], [8, 9, 10, 11, 12, -1, -1, -1],
                       [13, 14, 15, -1, -1, -1, -1, -1]], dtype=torch.int32)
    kp = torch.randint(0, 16, (3, 48), dtype=torch.int32)
    ca.check_lists(qp, kp, 16)
    kp[2, 0] = 16
    with pytest.raises(ca.ClusterAttnError, match="outside"):
        ca.check_lists(qp, kp, 16)


def test_binding_rejects_mismatched_shapes(lists):
    """Shape errors are raised before any device pointer is taken, so CPU
    tensors suffice to reach them."""
    q_idx, key_idx, N = lists
    x = torch.zeros(2, N, 4, 32, dtype=torch.bfloat16)
    lse = torch.zeros(2, N, 4)
    with pytest.raises(ValueError, match="key_idx"):
        ca.fwd(x, x, x, q_idx, key_idx[:1], 0.1)          # lists of another batch size
    with pytest.raises(ValueError, match="q_idx"):
        ca.fwd(x, x, x, q_idx[:, :100], key_idx, 0.1)     # too few clusters
    with pytest.raises(ValueError, match="q_idx"):
        ca.fwd(x[:, :1000], x[:, :1000], x[:, :1000], q_idx, key_idx[:, :125], 0.1)
    with pytest.raises(ValueError, match="lse"):
        ca.bwd(x, x, x, x, x, lse[:, :, :2], q_idx, key_idx, 0.1)
    with pytest.raises(ValueError, match="clusters"):
        ca.bwd_plan(q_idx, key_idx, N + 8)
    with pytest.raises(ValueError, match="q_idx"):
        ca.bwd_plan(q_idx[:1], key_idx, N)
