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


# ------------------------------------------------- trees of more than 64 nodes
def test_multiword_mask_chain_closed_form():
    # node i of a chain sees nodes 0..i: word w of row i holds min(64, i + 1 - 64 w) low bits
    T, W = 200, 4
    words = oracle.ancestor_or_self_words(list(range(-1, T - 1)), W)
    for i in range(T):
        for w in range(W):
            n = max(0, min(64, i + 1 - 64 * w))
            want = (1 << n) - 1 if n < 64 else (1 << 64) - 1
            assert int(words[i, w]) == want


def test_multiword_mask_matches_single_word_and_brute_force():
    import numpy as np
    rng = np.random.default_rng(5)
    for T in (1, 7, 64, 65, 130, 256):
        par = [-1] + [int(rng.integers(-1 if T % 2 else 0, i)) for i in range(1, T)]
        words = oracle.ancestor_or_self_words(par, 4)
        # brute force: walk up from every node
        for i in range(T):
            seen = set()
            j = i
            while j != -1:
                seen.add(j)
                j = par[j]
            got = {w * 64 + k for w in range(4) for k in range(64) if (int(words[i, w]) >> k) & 1}
            assert got == seen
        if T <= 64:
            single = oracle.ancestor_or_self_mask(par)
            assert np.array_equal(words[:, 0], single) and not words[:, 1:].any()
