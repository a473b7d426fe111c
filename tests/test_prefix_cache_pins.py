"""Pins of the oracle's prefix-cache models (CPU): the pages' worked
examples, brute-force longest-common-prefix reuse and the eviction order."""

import pytest

import cache_pins as P

HASH = P.hash_driver()
TREE = P.tree_driver()


@pytest.mark.parametrize("make", [HASH, TREE], ids=["hash", "tree"])
def test_ttft_example(make):
    P.pin_ttft(make)


def test_three_users_hash():
    P.pin_three_users(HASH)


def test_three_users_tree():
    P.pin_three_users(TREE, tree=True)


@pytest.mark.parametrize("make", [HASH, TREE], ids=["hash", "tree"])
def test_multi_turn_trace(make):
    P.pin_multi_turn(make)


def test_five_step_figure_hash():
    P.pin_five_step(HASH)


def test_five_step_figure_tree():
    P.pin_five_step(TREE, tree=True)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_lcp_hash(seed):
    P.pin_brute_force_lcp(HASH, seed, salts=True)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_lcp_tree(seed):
    P.pin_brute_force_lcp(TREE, seed)


def test_salt_separates_tenants():
    P.pin_salt(HASH)


def test_lru_order_hash():
    P.pin_lru_order(HASH, (4, 8))


def test_lru_order_tree():
    P.pin_lru_order(TREE, (0, 8))


def test_tree_never_evicts_held_or_inner_nodes():
    P.pin_tree_holds(TREE)


def test_hash_model_copies_before_writing_a_cached_block():
    P.pin_cached_block_copied()
