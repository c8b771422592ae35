"""The read-ceiling instruments of libpa_ceiling.so read exactly the pages
they are given: each wavefront folds every 32-bit word of its pages' K and V
into one sink word with xor, so the sink is checked bit for bit against the
same fold on the host."""
import numpy as np
import pytest
import torch

import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import ceiling
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def built():
    pa.ensure_built()


def caches(NB, KH, page_bytes, seed):
    g = torch.Generator().manual_seed(seed)
    words = page_bytes // 4
    kc = torch.randint(-2**31, 2**31 - 1, (NB, KH, words), dtype=torch.int32, generator=g)
    vc = torch.randint(-2**31, 2**31 - 1, (NB, KH, words), dtype=torch.int32, generator=g)
    return kc, vc


def fold(kc, vc, items):
    """xor of every word of the K and V pages (block, kv head) in `items`."""
    x = np.uint32(0)
    for b, h in items:
        x ^= np.bitwise_xor.reduce(kc[b, h].numpy().view(np.uint32))
        x ^= np.bitwise_xor.reduce(vc[b, h].numpy().view(np.uint32))
    return int(x)


@pytest.mark.parametrize("page_bytes", [2048, 4096])
def test_flat_gather_reads_exactly_its_pages(page_bytes):
    NB, KH = 48, 2
    kc, vc = caches(NB, KH, page_bytes, seed=page_bytes)
    blocks = torch.tensor([5, 0, 47, 12, 12, 33, 7, 21, 40, 2, 19], dtype=torch.int32)
    U.note(f"flat gather {page_bytes}")
    sink = torch.zeros(ceiling.sink_words(), dtype=torch.int32, device=U.DEV)
    ceiling.gather_ceiling(sink, kc.to(U.DEV), vc.to(U.DEV), blocks.to(U.DEV))
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    items = [(int(blocks[i // KH]), i % KH) for i in range(len(blocks) * KH)]
    waves = len(got)
    per = -(-len(items) // waves)
    want = np.zeros(waves, dtype=np.uint32)
    for w in range(waves):
        run = items[w * per:(w + 1) * per]
        if run:
            want[w] = fold(kc, vc, run)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("page_bytes,wgs", [(4096, 2), (2048, 3)])
def test_unit_gather_reads_exactly_its_units(page_bytes, wgs):
    NB, KH, BS = 40, 2, 16
    kc, vc = caches(NB, KH, page_bytes, seed=7 + page_bytes)
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(3)).to(torch.int32)
    lens = torch.tensor([0, 130, 16, 200, 1], dtype=torch.int32)
    nb = (lens + BS - 1) // BS
    bt = torch.full((len(lens), 13), -1, dtype=torch.int32)
    used = 0
    for s, n in enumerate(nb.tolist()):
        bt[s, :n] = perm[used:used + n]
        used += n
    pages, off, n = ceiling.unit_pages(bt, lens, BS, KH, 4)
    assert n > 0 and int(off[-1]) == int(nb.sum()) * KH
    U.note(f"unit gather {page_bytes} wgs={wgs} units={n}")
    sink = torch.zeros(4 * n, dtype=torch.int32, device=U.DEV)
    ceiling.gather_units(sink, kc.to(U.DEV), vc.to(U.DEV), pages.to(U.DEV), off.to(U.DEV), n, wgs)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32).reshape(n, 4)
    for u in range(n):
        unit = pages[off[u]:off[u + 1]].tolist()
        for w in range(4):
            items = [(p // KH, p % KH) for p in unit[w::4]]
            assert int(got[u, w]) == fold(kc, vc, items), (u, w)
