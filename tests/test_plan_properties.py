"""Property tests of the host-side planner over random shapes (no GPU): the schedule the
library picks must cover every token and vocabulary row, keep the gradient block within the
chunk bound, keep every operand a tile addresses below 2 GiB (32-bit offsets), and keep the
workspace independent of T x V."""
import pytest
from hypothesis import given, settings, strategies as st

I32 = (1 << 31) - 1


@pytest.fixture(scope="module")
def flce():
    from chunked_lm_head_amd import flce as m
    return m


shapes = st.tuples(
    st.integers(1, 1 << 20),                                   # T
    st.integers(1, 8192).map(lambda d: d * 8),                 # D, a multiple of 8
    st.integers(1, 1 << 20),                                   # V
    st.integers(1, 4096),                                      # chunk_rows
)


@settings(max_examples=400, deadline=None)
@given(shapes)
def test_cross_entropy_plan_invariants(flce, shape):
    T, D, V, cr = shape
    p = flce.describe_plan(T, D, V, cr)
    R, Vc = p["row_block"], p["vocab_chunk"]
    assert R % 256 == 0 and Vc % 256 == 0 and R >= 256 and Vc >= 256
    # every token and vocabulary row is covered, and no block / chunk is wholly empty
    assert R * p["row_blocks"] >= T and (p["row_blocks"] - 1) * R < T
    assert Vc * p["vocab_chunks"] >= V and (p["vocab_chunks"] - 1) * Vc < V
    assert p["token_tiles"] == -(-T // 256) and p["vocab_tiles"] == -(-V // 256)
    assert 1 <= p["fwd_splits"] <= p["vocab_tiles"]
    # the bf16 gradient block stays within one chunk of fp32 logits (at least one tile)
    assert p["grad_tile_bytes"] == R * Vc * 2
    assert p["grad_tile_bytes"] <= max(cr * V * 4, 256 * 256 * 2)
    assert R <= 8192
    # 32-bit tile addressing: the gradient block and the lm_head rows of one chunk stay
    # below 2 GiB, unless a single vocabulary tile is already past that
    assert R * Vc * 2 <= I32 or Vc == 256
    assert Vc * D * 2 <= I32 or Vc == 256
    assert p["dh_splits"] >= 1
    assert p["dh_splits"] * R * D * 4 <= max(R * D * 4, 128 << 20)
    ws = flce.workspace_bytes(T, D, V, cr)
    assert ws >= max(p["fwd_workspace"], p["bwd_workspace"])


@settings(max_examples=300, deadline=None)
@given(shapes)
def test_workspace_is_one_chunk_block_plus_linear_terms(flce, shape):
    """The workspace holds one gradient block (within the chunk bound), per-token arrays and
    forward partial sums (O(T)), and the dH partial sums and staged hidden rows of one row
    block (O(R D)): no term in T x V."""
    T, D, V, cr = shape
    ws = flce.workspace_bytes(T, D, V, cr)
    block = max(cr * V * 4, 256 * 256 * 2)
    linear = 32 * (T + 256) + (8 << 20) + (128 << 20) + 6 * 8192 * D
    assert ws <= block + linear, (T, D, V, cr, ws)


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 1 << 18), st.integers(1, 2048).map(lambda d: d * 8),
       st.integers(1, 2048).map(lambda d: d * 8), st.integers(1, 1 << 18), st.integers(1, 1024))
def test_distill_workspace_within_the_chunk_bound(flce, T, Ds, Dt, V, cr):
    n = flce.distill_workspace_bytes(T, Ds, Dt, V, cr)
    R_max = 8192
    # the fp32 p_t block (G over it) within one chunk of fp32 logits (at least one tile),
    # plus O(T) per-token arrays, per-workgroup partial sums, the forward's partials, the
    # student's dH partial sums (split-K sums capped at 128 MiB, or one row block's) and
    # its H^T (O(R D))
    block = max(cr * V * 4, 256 * 256 * 4)
    dh_sums = max(R_max * max(Ds, 8) * 4, 128 << 20)
    linear = (64 * (T + R_max) + 2 * 4 * V * 64 + dh_sums + R_max * max(Ds, 8) * 2
              + (8 << 20))
    assert 0 < n <= block + linear, (T, Ds, Dt, V, cr, n)


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 4096), st.integers(1, 64), st.integers(1, 512).map(lambda d: d * 8),
       st.integers(1, 1 << 17), st.integers(1, 512))
def test_policy_workspace_is_the_cross_entropy_one_plus_per_token_arrays(flce, S, n_seq, D, V,
                                                                         cr):
    T = S * n_seq
    base = flce.workspace_bytes(T, D, V, cr)
    got = flce.policy_workspace_bytes(T, D, V, cr, n_seq)
    assert base + 12 * T + 16 * n_seq <= got <= base + 12 * T + 16 * n_seq + 7 * 256
    # equal-length sequences only: T must split evenly into n_seq of them
    bad_T, bad_n = (T + 1, n_seq) if n_seq > 1 else (T, T + 1)
    with pytest.raises(ValueError):
        flce.policy_workspace_bytes(bad_T, D, V, cr, bad_n)


@settings(max_examples=200, deadline=None)
@given(st.integers(-4, 1 << 20), st.integers(-8, 1 << 17), st.integers(-4, 1 << 20),
       st.integers(-4, 4096))
def test_invalid_shapes_are_refused(flce, T, D, V, cr):
    """Negative T, non-positive D / V / chunk_rows, D not a multiple of 8 or D above 65,536
    yield no plan and no workspace size."""
    valid = T >= 0 and D >= 1 and V >= 1 and cr >= 1 and D % 8 == 0 and D <= 1 << 16
    if valid:
        assert flce.workspace_bytes(T, D, V, cr) > 0
        flce.describe_plan(T, D, V, cr)
    else:
        with pytest.raises(ValueError):
            flce.workspace_bytes(T, D, V, cr)
        with pytest.raises(Exception):
            flce.describe_plan(T, D, V, cr)
