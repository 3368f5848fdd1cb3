"""Pins for the oracle's tree mask (CPU only)."""
import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from helpers import dp_masks, read_mask_table


@pytest.mark.parametrize("name,parents,words", read_mask_table())
def test_mask_golden_tables(name, parents, words):
    got = oracle.ancestor_or_self_mask(parents)
    assert [int(x) for x in got] == words, name


@st.composite
def trees(draw):
    T = draw(st.integers(1, 64))
    par = [-1]
    for i in range(1, T):
        par.append(draw(st.integers(-1, i - 1)))
    return par


@settings(max_examples=200, deadline=None)
@given(trees())
def test_mask_walk_matches_parent_combination(par):
    assert [int(x) for x in oracle.ancestor_or_self_mask(par)] == dp_masks(par)


def test_mask_chain64_closed_form():
    # a 64-node chain: node i sees 0..i, i.e. word 2^(i+1) - 1
    par = [-1] + list(range(63))
    got = [int(x) for x in oracle.ancestor_or_self_mask(par)]
    assert got == [(1 << (i + 1)) - 1 for i in range(64)]


def test_mask_properties_random():
    rng = np.random.default_rng(7)
    for _ in range(50):
        T = int(rng.integers(1, 65))
        par = [-1] + [int(rng.integers(-1, i)) for i in range(1, T)]
        m = [int(x) for x in oracle.ancestor_or_self_mask(par)]
        for i in range(T):
            assert m[i] >> i & 1                     # self
            assert m[i] >> (i + 1) == 0              # never a later node
            if par[i] >= 0:                          # parent's set plus self
                assert m[i] == m[par[i]] | (1 << i)
            else:
                assert m[i] == 1 << i


@pytest.mark.parametrize("bad", [[0], [-1, 1], [-1, 0, 3], [-1, -2], [-1, 0, 2]])
def test_mask_rejects_bad_parents(bad):
    with pytest.raises(ValueError):
        oracle.ancestor_or_self_mask(bad)


def test_mask_rejects_more_than_64_nodes():
    with pytest.raises(ValueError):
        oracle.ancestor_or_self_mask([-1] + list(range(64)))
