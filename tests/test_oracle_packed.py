"""Pins for the packed-weight oracle (CPU only).

The layout is defined in oracle/packed.py by a position formula. It is pinned
three ways, each independent of how the oracle evaluates that formula:
  * it is a bijection onto range(N*K) (the repack moves bytes, never drops or
    duplicates one);
  * every packed byte, decoded position -> (block, lane, byte) -> (n, k) by
    plain integer arithmetic in the other direction, holds qw[n, k];
  * the operand contract it exists for: a loop emulating the 16x16x64 INT8
    matrix instruction (lane l supplies row l % 16 and K positions
    16*(l // 16) .. +15 of both operands, the 64 products of a row-column pair
    summed) over the packed weights and the row-major activations reproduces
    the exact per-group partial sums q[:, group] @ qw[:, group].T.
A layout with rows and lanes transposed, or the K quarters in the wrong lanes,
fails the last two (checked below on planted mistakes).
"""
import numpy as np
import pytest

from oracle import group_partials_ref, packed_position_ref, repack_mfma_ref, unpack_mfma_ref


def _qw(N, K, seed=0):
    return np.random.default_rng(seed).integers(-127, 128, (N, K), dtype=np.int8)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (1024, 7168), (272, 1152)])
def test_positions_are_a_permutation(N, K):
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    pos = np.sort(packed_position_ref(n, k, K).ravel())
    assert np.array_equal(pos, np.arange(N * K))


def _decode_position(p, K):
    """(n, k) stored at packed byte p, decoded from the block / lane / byte split."""
    block, within = divmod(p, 1024)
    nb, s = divmod(block, K // 64)
    lane, j = divmod(within, 16)
    return 16 * nb + lane % 16, 64 * s + 16 * (lane // 16) + j


@pytest.mark.parametrize("N,K", [(16, 128), (32, 256), (48, 384)])
def test_every_packed_byte_decodes_to_its_source(N, K):
    qw = _qw(N, K, N + K)
    packed = repack_mfma_ref(qw)
    for p in range(N * K):
        n, k = _decode_position(p, K)
        assert packed[p] == qw[n, k], p
    assert np.array_equal(unpack_mfma_ref(packed, N, K), qw)


def _mfma_group_partials(q, packed, N, K):
    """P[m, n, g] computed the way a 16x16x64 INT8 instruction consumes the packed
    weights: for each 16-row block and 64-wide K step, lane l of the weight
    operand is packed bytes [16l, 16l+16) of the block, lane l of the activation
    operand row l % 16 of q at K positions 64s + 16*(l // 16) .. +15; the
    instruction sums over its 64 K positions, two instructions make a group."""
    M = q.shape[0]
    G = K // 128
    P = np.zeros((M, N, G), np.int64)
    blk = np.asarray(packed).reshape(N // 16, K // 64, 64, 16).astype(np.int64)
    for nb in range(N // 16):
        for s in range(K // 64):
            for c in range(16):            # output column = weight row 16*nb + c
                for quarter in range(4):   # the four lanes carrying column c
                    l = c + 16 * quarter
                    wbytes = blk[nb, s, l]
                    k0 = 64 * s + 16 * quarter
                    P[:, 16 * nb + c, s // 2] += q[:, k0:k0 + 16].astype(np.int64) @ wbytes
    return P


@pytest.mark.parametrize("M,N,K", [(16, 32, 256), (5, 48, 384)])
def test_operand_contract_gives_the_group_partials(M, N, K):
    rng = np.random.default_rng(M * N)
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = _qw(N, K, 7)
    P = _mfma_group_partials(q, repack_mfma_ref(qw), N, K)
    assert np.array_equal(P, group_partials_ref(q, qw).astype(np.int64))


def test_planted_layout_mistakes_fail_the_pins():
    """Two plausible slips, planted in a copy of the layout on the CPU: the
    column and K-quarter roles of the lane swapped, and rows transposed with
    columns inside a block. Both must break the operand-contract pin."""
    M, N, K = 16, 32, 256
    rng = np.random.default_rng(3)
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    qw = _qw(N, K, 11)
    want = group_partials_ref(q, qw).astype(np.int64)
    n, k = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")

    def pack_with(pos):
        out = np.zeros(N * K, np.int8)
        out[pos.ravel()] = qw.ravel()
        return out

    lane_swapped = 4 * (n % 16) + (k % 64) // 16          # column and quarter roles swapped
    pos1 = ((n // 16) * (K // 64) + k // 64) * 1024 + 16 * lane_swapped + k % 16
    transposed = ((n // 16) * (K // 64) + k // 64) * 1024 + (k % 64) * 16 + n % 16
    for pos in (pos1, transposed):
        assert np.array_equal(np.sort(pos.ravel()), np.arange(N * K))   # still permutations
        assert not np.array_equal(_mfma_group_partials(q, pack_with(pos), N, K), want)
