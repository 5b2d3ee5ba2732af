"""GPU parity of the prefix-aware decode (kvq_decode_prefix_attention)
through the C ABI.

The member sequences of a group hold the same tokens over a common prefix
and, after the cache is built, their block tables point at the first
member's physical pages for it (OSCAR technical summary, sec. 2.2-B: paged
attention with prefix caching).  The prefix-aware decode reads those pages
once per row set of four members; its outputs must match the oracle's
decode of the same cache within 2e-3, and the plain decode's within the
same bound (the two differ only in where the split-K boundaries fall,
which moves outputs by up to ~1e-4 here and ~1e-3 on the 64-sequence
workload).  Cases cover five members (two
row sets), single-member groups, an empty group, a member whose INT2 tiles
do not reach the prefix, a sequence listed twice, prefixes that end inside a
tile, no groups, and G = 1, 2, 4, 8 query heads per KV head."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, Scenario, dev_u16, rel_err, say
from long_context_decode_kvq_amd import kvq2
from long_context_decode_kvq_amd.workloads import normal_bits

pytestmark = pytest.mark.gpu

CASES = [
    # id, (Hq, Hkv, P, n_sink, W), lens, groups [(members, prefix tokens)]
    ("g4_rowsets", (8, 2, 16, 4, 32), [900, 700, 1000, 650, 800, 300],
     [([0, 1, 2, 3, 4], 512)]),
    ("g8_two_groups", (16, 2, 32, 0, 64), [1200, 1100, 1300, 900],
     [([0, 1], 640), ([2], 320)]),
    ("g2_short_member", (4, 2, 64, 20, 16), [1500, 1100, 600],
     [([0, 1, 2], 1024)]),
    ("g4_duplicate_empty", (8, 2, 16, 4, 32), [700, 720, 760, 400],
     [([0, 1], 512), ([], 256), ([1, 2], 512)]),
    ("g4_ragged_prefix", (8, 4, 16, 4, 8), [500, 530, 610],
     [([2, 0, 1], 496)]),
    ("g1_heads", (2, 2, 16, 4, 16), [800, 820],
     [([1, 0], 480)]),
    ("g4_batch1", (8, 2, 16, 4, 32), [1000], [([0], 768)]),
    ("no_groups", (8, 2, 16, 4, 32), [600, 500], []),
]


def _share(sc: Scenario, groups):
    """Give each group's members the first member's tokens over the prefix,
    build the cache, then point the members' block tables at the first
    member's pages for the whole pages the prefix covers (within each
    member's length)."""
    P = sc.od.page_size
    for members, plen in groups:
        if not members:
            continue
        b0 = members[0]
        for b in members[1:]:
            n = min(plen, sc.lens[b], sc.lens[b0])
            sc.k_all[b][:n] = sc.k_all[b0][:n]
            sc.v_all[b][:n] = sc.v_all[b0][:n]
    sc.fill_to(pieces=2)
    bt = sc.dc.block_table.clone()
    seen = set()
    for members, plen in groups:
        if not members:
            continue
        b0 = members[0]
        for b in members[1:]:
            if b in seen or b == b0:
                continue
            npg = min(plen, sc.lens[b], sc.lens[b0]) // P
            bt[b, :npg] = bt[b0, :npg]
        seen.update(members)
    sc.dc.block_table.copy_(bt)


def _groups(groups):
    starts = np.zeros(len(groups) + 1, np.int32)
    for j, (members, _) in enumerate(groups):
        starts[j + 1] = starts[j] + len(members)
    members = np.array([b for m, _ in groups for b in m] or [0], np.int32)
    plen = np.array([p for _, p in groups] or [0], np.int32)
    t = [torch.from_numpy(x).cuda() for x in (starts, members, plen)]
    if not groups:
        return kvq2.prefix_groups(0), t
    return kvq2.prefix_groups(int(starts[-1]), *t), t


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefix_decode_matches_oracle(case):
    name, (Hq, Hkv, P, ns, W), lens, groups = case
    say(f"[prefix] {name}: heads {Hq}/{Hkv} P={P} sink={ns} W={W} lens={lens} groups={groups}")
    sc = Scenario(Hq, Hkv, P, ns, W, lens, seed=11 + len(lens) + Hq)
    _share(sc, groups)
    out_plain, ref, _ = sc.decode()
    q = normal_bits(sc.seed * 31 + 99, (sc.B, Hq, 128))
    seq = torch.tensor(sc.cur, dtype=torch.int32, device="cuda")
    maxL = max(sc.cur)
    g, keep = _groups(groups)
    nbytes = kvq2.decode_prefix_workspace_bytes(sc.kd, sc.B, maxL, g)
    assert nbytes >= kvq2.decode_workspace_bytes(sc.kd, sc.B, maxL)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((sc.B, Hq, 128), float("nan"), device="cuda")
    for _ in range(2):   # the workspace is reused
        kvq2.decode_prefix_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, maxL, dev_u16(q),
                                     out, g, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        e, d = rel_err(got, ref), rel_err(got, out_plain)
        say(f"  rel_err vs oracle {e:.2e}, vs plain decode {d:.2e}")
        assert e <= TOL
        assert d <= TOL
    del keep


@pytest.mark.parametrize("heads", [(8, 2), (16, 2)], ids=["g4", "g8"])
def test_group_tiles_are_read_through_the_group(heads):
    """The group's prefix tiles come from its representative's pages, not the
    member's own: with private, different pages under a declared group, the
    prefix-aware decode matches an oracle whose members read the first
    member's pages over the prefix tiles (512 positions = 8 pages of 64, no
    sink: exactly the group's whole tiles), and differs from the plain
    decode of the private pages."""
    Hq, Hkv = heads
    sc = Scenario(Hq, Hkv, 64, 0, 32, [900, 800, 1000, 760], seed=5 + Hq)
    sc.fill_to(pieces=2)
    out_plain, ref_private, _ = sc.decode()
    members = [0, 1, 3]
    bt = sc.oc.block_table.copy()
    for b in members[1:]:
        bt[b, :8] = bt[0, :8]
    sc.oc.block_table[:] = bt
    q = normal_bits(sc.seed * 31 + 99, (sc.B, Hq, 128))
    ref_shared = sc.oc.decode(sc.R_K, sc.R_V, sc.cur, q)
    g, keep = _groups([(members, 512)])
    seq = torch.tensor(sc.cur, dtype=torch.int32, device="cuda")
    maxL = max(sc.cur)
    ws = torch.zeros(kvq2.decode_prefix_workspace_bytes(sc.kd, sc.B, maxL, g), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((sc.B, Hq, 128), float("nan"), device="cuda")
    kvq2.decode_prefix_attention(sc.kd, sc.layer, sc.dc.handle, sc.B, seq, maxL, dev_u16(q), out,
                                 g, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    e_shared, e_private = rel_err(got, ref_shared), rel_err(got[members[1:]], ref_private[members[1:]])
    say(f"  vs shared-page oracle {e_shared:.2e}, members vs private pages {e_private:.2e}")
    assert e_shared <= TOL
    assert e_private > 20 * TOL
    assert rel_err(got[[0, 2]], out_plain[[0, 2]]) <= TOL
    del keep
