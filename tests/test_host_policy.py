"""Host policy of the library (no device call): rows per chunk from the page's
chunk multiplier, and the choice of mini-batches and chunk size for a memory
budget."""
import math

import pytest

from oracle import flce_oracle as o


@pytest.fixture(scope="module")
def flce():
    from chunked_lm_head_amd import flce as m
    return m


# the page's default multiplier max(4, context // 4096), evaluated by hand
HAND_MULTIPLIER = {1: 4, 100: 4, 4095: 4, 4096: 4, 8192: 4, 16383: 4, 16384: 4, 20000: 4,
                   24576: 6, 64000: 15, 65536: 16, 131072: 32, 1 << 20: 256}


@pytest.mark.parametrize("ctx", sorted(HAND_MULTIPLIER))
def test_default_chunk_rows_follow_the_page_multiplier(flce, ctx):
    mult = HAND_MULTIPLIER[ctx]
    assert flce.chunk_rows_for(ctx) == math.ceil(ctx / mult)
    assert flce.chunk_rows_for(ctx, 0) == flce.chunk_rows_for(ctx, -5)


def test_page_example_chunks(flce):
    # batch 4 x context 8192 x vocab 128,000: multiplier 4, 16 chunks of 2048 rows;
    # Equation 3's logit memory of one chunk is chunk_rows x vocab elements
    batch, ctx, vocab = 4, 8192, 128000
    mult = o.default_multiplier(ctx)
    rows = flce.chunk_rows_for(ctx)
    assert (mult, rows, batch * mult * rows) == (4, 2048, batch * ctx)
    assert o.logit_memory_eq3(ctx, vocab, mult) * 1024 ** 3 == rows * vocab


def test_explicit_multiplier(flce):
    assert flce.chunk_rows_for(1000, 3) == 334
    assert flce.chunk_rows_for(1000, 1) == 1000
    assert flce.chunk_rows_for(1000, 5000) == 1
    with pytest.raises(ValueError):
        flce.chunk_rows_for(0)


def _need(flce, batch, ctx, D, V, m, cr):
    tmb = -(-batch // m) * ctx
    return flce.workspace_bytes(tmb, D, V, cr) + tmb * D * 4 + tmb * 16


@pytest.mark.parametrize("batch,ctx,D,V,budget", [
    (4, 8192, 4096, 128000, 64 << 30),
    (4, 8192, 4096, 128000, 300 << 20),
    (8, 64000, 4096, 151936, 2 << 30),
    (3, 5000, 2048, 248320, 1 << 30),
    (1, 131072, 4096, 151936, 4 << 30),
])
def test_tune_fits_and_is_minimal(flce, batch, ctx, D, V, budget):
    r = flce.tune(batch, ctx, D, V, budget)
    m, cr = r["mini_batches"], r["chunk_rows"]
    assert r["bytes_needed"] == _need(flce, batch, ctx, D, V, m, cr) <= budget
    default_rows = flce.chunk_rows_for(ctx)
    assert cr <= default_rows
    # the next larger chunk (multiplier one smaller, not below the default) does not fit
    if cr < default_rows:
        k = -(-ctx // cr)                       # smallest multiplier giving cr rows
        while -(-ctx // (k - 1)) == cr:
            k -= 1
        assert k - 1 >= o.default_multiplier(ctx)
        bigger = flce.chunk_rows_for(ctx, k - 1)
        assert bigger > cr and _need(flce, batch, ctx, D, V, m, bigger) > budget
    # fewer mini-batches (a larger group) do not fit at any chunk size tried
    if m > 1:
        bigger = [k for k in range(1, m) if -(-batch // k) > -(-batch // m)]
        for k in bigger[-1:]:
            assert _need(flce, batch, ctx, D, V, k, 1) > budget or \
                all(_need(flce, batch, ctx, D, V, k, c) > budget
                    for c in (1, default_rows))


def test_tune_huge_budget_keeps_defaults(flce):
    r = flce.tune(4, 8192, 4096, 128000, 1 << 40)
    assert (r["mini_batches"], r["chunk_rows"]) == (1, 2048)


def test_tune_errors(flce):
    with pytest.raises(flce.FlceError) as e:
        flce.tune(4, 8192, 4096, 128000, 1 << 20)
    assert e.value.status == 3
    with pytest.raises(flce.FlceError) as e:
        flce.tune(0, 8192, 4096, 128000, 1 << 30)
    assert e.value.status == 2
    with pytest.raises(flce.FlceError) as e:
        flce.tune(4, 8192, 4090, 128000, 1 << 30)
    assert e.value.status == 4
