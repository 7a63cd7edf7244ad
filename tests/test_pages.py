"""Host-side page pool (attn_pages_*): invariants under random use.

The pages' description fixes what must hold, not which ids are handed out
("LLM 核心技术：Attention 机制的实现与优化", PagedAttention section: fixed-size
pages from one global pool, a per-sequence table of where its logical pages
live, pages returned when no longer needed). A plain Python model tracks the
expected lengths; the checks are: every sequence owns exactly
ceil(len / page_size) pages, no page is owned twice or both owned and free,
owned + free = num_pages, a request that does not fit fails and changes
nothing, shrinking keeps the logical prefix of pages, and the table is the
sequences' page lists back to back in the requested order (the layout
oracle.sequence_pages describes).
"""

import os
import random

import pytest

import oracle
import scaled_dot_product_flash_amd as attn


@pytest.fixture(scope="module")
def built():
    if not os.path.exists(attn.library_path()):
        pytest.skip("libattn.so not built")
    attn.load_library()


def _check_state(pool, model, ps):
    ids = sorted(model)
    table, lens = pool.table(ids)
    assert lens.tolist() == [model[i] for i in ids]
    counts = [(n + ps - 1) // ps for n in lens.tolist()]
    assert len(table) == sum(counts)
    owned = table.tolist()
    assert len(set(owned)) == len(owned)
    assert all(0 <= p < pool.num_pages for p in owned)
    assert pool.free_count() + len(owned) == pool.num_pages
    # the ragged layout: sequence i owns entries first_i .. first_i + count_i - 1
    assert [c for _, c in oracle.sequence_pages(lens.tolist(), ps)] == counts
    return {i: owned[f:f + c] for i, (f, c) in zip(ids, oracle.sequence_pages(lens.tolist(), ps))}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_resizes_keep_invariants(built, seed):
    rng = random.Random(seed)
    ps, num_pages = 16, 64
    pool = attn.PagePool(num_pages, ps)
    model = {}
    pages = {}
    for _ in range(400):
        sid = rng.randrange(12)
        new = rng.choice([0, rng.randrange(1, 40), rng.randrange(1, 300), model.get(sid, 0) + 1])
        have = (model.get(sid, 0) + ps - 1) // ps
        need = (new + ps - 1) // ps
        free_before = pool.free_count()
        if need - have > free_before:
            with pytest.raises(RuntimeError, match="-11"):
                pool.resize(sid, new)
            after = _check_state(pool, model, ps)
            assert after == pages  # a failed request changes nothing
            continue
        pool.resize(sid, new)
        if new == 0:
            model.pop(sid, None)
        else:
            model[sid] = new
        after = _check_state(pool, model, ps)
        if sid in pages and sid in after:
            keep = min(len(pages[sid]), len(after[sid]))
            assert after[sid][:keep] == pages[sid][:keep]  # logical pages never move
        pages = after
    pool.close()


def test_freed_pages_are_reused_and_order_is_requested_order(built):
    pool = attn.PagePool(6, 8)
    pool.resize(1, 17)   # 3 pages
    pool.resize(2, 8)    # 1 page
    pool.resize(3, 9)    # 2 pages
    assert pool.free_count() == 0
    t_a, l_a = pool.table([3, 1, 2])
    t_b, l_b = pool.table([1, 2, 3])
    assert l_a.tolist() == [9, 17, 8] and l_b.tolist() == [17, 8, 9]
    assert sorted(t_a.tolist()) == sorted(t_b.tolist()) == list(range(6))
    pool.resize(1, 0)    # release all of sequence 1
    assert pool.free_count() == 3
    pool.resize(4, 24)   # takes exactly the three released pages
    t, _ = pool.table([4])
    assert sorted(t.tolist()) == sorted(t_b[:3].tolist())
    with pytest.raises(RuntimeError, match="-12"):
        pool.table([1])
    pool.close()
