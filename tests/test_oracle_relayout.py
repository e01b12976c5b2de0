"""Pins for the oracle's relayout, padding and spatial routines (CPU only).

Each check is tied to something other than the oracle itself: hand-written
fixtures from the pages' diagrams, a torch permute that expresses the same
map through library reshapes, round trips, coordinate decoding, and the
world-size-1 identity route.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _labels_to_codes(nested, table):
    if isinstance(nested, str):
        if nested not in table:
            table[nested] = len(table) + 1
        return table[nested]
    return [_labels_to_codes(n, table) for n in nested]


@pytest.mark.parametrize("fixture", ["scatter_p2_labels.json", "scatter_p4_h8_labels.json"])
def test_golden_label_fixtures(orc, fixture):
    """Hand-written relayouts from the Ulysses diagram (TeleFuser 'Communication
    Architecture', 'Ulysses'; flashinfer #6332 'Description')."""
    g = json.load(open(os.path.join(GOLDEN, fixture)))
    table = {}
    x = np.array(_labels_to_codes(g["input"], table), dtype=np.uint16)[..., None]
    want = np.array(_labels_to_codes(g["scatter_output"], table), dtype=np.uint16)[..., None]
    assert x.shape == (g["P"], g["B"], g["S_local"], g["H"], g["D"])
    y = orc.scatter(x)
    np.testing.assert_array_equal(y, want)
    np.testing.assert_array_equal(orc.gather(y), x)


def _torch_scatter(x: np.ndarray) -> np.ndarray:
    """Library special case: the same map via torch view/permute/reshape."""
    P, B, S_l, H, D = x.shape
    t = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x)
    t = t.view(P, B, S_l, P, H // P, D).permute(3, 1, 0, 2, 4, 5).reshape(P, B, P * S_l, H // P, D)
    out = t.contiguous().numpy()
    return out.view(x.dtype)


SHAPES = [
    # P, B, S_l, H, D
    (1, 1, 3, 4, 8),
    (2, 1, 5, 4, 8),
    (2, 2, 7, 8, 64),
    (3, 2, 5, 6, 4),
    (4, 1, 9, 8, 16),
    (4, 1, 200, 4, 128),   # tail row count used by flashinfer #6332's tests
    (8, 2, 3, 16, 8),
    (8, 1, 2, 8, 128),     # one head per rank (GQA K/V band)
]


@pytest.mark.parametrize("shape", SHAPES)
def test_scatter_matches_torch_permute(orc, shape):
    rng = np.random.default_rng(sum(shape))
    x = rng.integers(0, 2 ** 16, size=shape, dtype=np.uint16)
    np.testing.assert_array_equal(orc.scatter(x), _torch_scatter(x))


@pytest.mark.parametrize("shape", SHAPES)
def test_round_trips(orc, shape):
    P, B, S_l, H, D = shape
    rng = np.random.default_rng(7 + sum(shape))
    x = rng.integers(0, 2 ** 16, size=shape, dtype=np.uint16)
    np.testing.assert_array_equal(orc.gather(orc.scatter(x)), x)
    o = rng.integers(0, 2 ** 16, size=(P, B, P * S_l, H // P, D), dtype=np.uint16)
    np.testing.assert_array_equal(orc.scatter(orc.gather(o)), o)


def test_coordinate_decoding(orc):
    """Every output word decodes to the source coordinate the Ulysses map names."""
    P, B, S_l, H, D = 4, 2, 6, 8, 4
    idx = np.arange(P * B * S_l * H * D, dtype=np.int64).reshape(P, B, S_l, H, D)
    y = orc.scatter(idx)            # int64 payload: unique codes, opaque copy
    Hl = H // P
    for q, b, gpos, j, d in itertools.product(range(P), range(B), range(P * S_l), range(Hl), range(D)):
        code = int(y[q, b, gpos, j, d])
        r, rem = divmod(code, B * S_l * H * D)
        bb, rem = divmod(rem, S_l * H * D)
        s, rem = divmod(rem, H * D)
        h, dd = divmod(rem, D)
        # source token s of rank r sits at global row r*S_l + s; head band q
        assert (bb, r * S_l + s, h, dd) == (b, gpos, q * Hl + j, d)


def test_world_size_one_is_identity(orc):
    """flashinfer UlyssesCommunicator PR, 'What': world size 1 is the identity route."""
    rng = np.random.default_rng(3)
    x = rng.integers(0, 2 ** 16, size=(1, 2, 5, 3, 8), dtype=np.uint16)
    np.testing.assert_array_equal(orc.scatter(x)[0], x[0])
    np.testing.assert_array_equal(orc.gather(x)[0], x[0])


def test_bit_patterns_and_multiset_preserved(orc):
    """Opaque bytes: NaN payloads, -0, subnormals pass unchanged; no word is lost."""
    special = np.array([0x7FC1, 0xFFFF, 0x8000, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x3F80], np.uint16)
    rng = np.random.default_rng(11)
    x = rng.choice(special, size=(2, 1, 4, 4, 8)).astype(np.uint16)
    y = orc.scatter(x)
    assert sorted(y.ravel().tolist()) == sorted(x.ravel().tolist())
    np.testing.assert_array_equal(y, _torch_scatter(x))


def test_divisibility_refused(orc):
    """'Ulysses': heads divisible by the world size; gathered sequence divisible on the inverse."""
    with pytest.raises(ValueError):
        orc.scatter(np.zeros((3, 1, 2, 4, 2), np.uint16))
    with pytest.raises(ValueError):
        orc.gather(np.zeros((2, 1, 3, 2, 2), np.uint16))


# ---------------------------------------------------------------------------
# padding / restoration of a non-divisible sequence
# ---------------------------------------------------------------------------
def test_padded_local_len_long_sequence(orc):
    # 75600 tokens over 4 ranks with a 128-token tile -> 75776 = 4 * 18944
    assert orc.padded_local_len(75600, 4, 128) == 18944
    for tile in (64, 128, 256):
        assert orc.padded_local_len(75600, 4, tile) * 4 == 75776
    assert orc.padded_local_len(512, 4, 128) == 128


@pytest.mark.parametrize("P,B,S,R,tile", [(4, 1, 75, 6, 8), (2, 2, 13, 4, 4), (3, 1, 10, 2, 1)])
def test_pad_shard_trim_round_trip(orc, P, B, S, R, tile):
    rng = np.random.default_rng(P * 100 + S)
    full = rng.integers(1, 2 ** 16, size=(B, S, R), dtype=np.uint16)
    S_l = orc.padded_local_len(S, P, tile)
    x = orc.pad_shard(full, P, S_l)
    assert x.shape == (P, B, S_l, R)
    # shard r holds global rows [r*S_l, (r+1)*S_l), zero past S
    flat = np.concatenate([x[r] for r in range(P)], axis=1)
    np.testing.assert_array_equal(flat[:, :S], full)
    assert (flat[:, S:] == 0).all()
    np.testing.assert_array_equal(orc.unshard_trim(x, S), full)
    # the whole exchange on a padded sequence restores the input
    H, D = 4, 2
    full5 = rng.integers(1, 2 ** 16, size=(B, S, H * P, D), dtype=np.uint16)
    xs = orc.pad_shard(full5, P, S_l)
    back = orc.unshard_trim(orc.gather(orc.scatter(xs)), S)
    np.testing.assert_array_equal(back, full5)


# ---------------------------------------------------------------------------
# height-sharded spatial tensors
# ---------------------------------------------------------------------------
def test_height_split_matches_array_split(orc):
    for Hh, P in [(90, 4), (7, 3), (8, 4), (5, 8)]:
        h, o = orc.height_split(Hh, P)
        parts = np.array_split(np.arange(Hh), P)
        assert h.tolist() == [len(p) for p in parts]
        assert o.tolist() == [int(p[0]) if len(p) else int(sum(h[:i])) for i, p in enumerate(parts)]
    h, o = orc.height_split(90, 4)
    assert h.tolist() == [23, 23, 22, 22] and o.tolist() == [0, 23, 46, 68]


@pytest.mark.parametrize("shape,P", [((1, 2, 3, 10, 5), 4), ((2, 1, 1, 9, 3), 3), ((1, 1, 2, 90, 4), 4)])
def test_spatial_round_trip_and_halos(orc, shape, P):
    rng = np.random.default_rng(sum(shape))
    full = rng.integers(1, 2 ** 16, size=shape, dtype=np.uint16)
    Hh = shape[-2]
    h, o = orc.height_split(Hh, P)
    sh = orc.spatial_split_halo(full, P, halo=1)
    hmax = int(h.max())
    assert sh.shape == (P,) + shape[:-2] + (hmax + 2, shape[-1])
    for r in range(P):
        core = sh[r][..., 1:1 + h[r], :]
        np.testing.assert_array_equal(core, full[..., o[r]:o[r] + h[r], :])
        top, bot = sh[r][..., 0, :], sh[r][..., h[r] + 1, :]
        if r == 0:
            assert (top == 0).all()        # no neighbour above: zero halo
        else:
            np.testing.assert_array_equal(top, full[..., o[r] - 1, :])   # neighbour's edge row
        if r == P - 1:
            assert (bot == 0).all()
        else:
            np.testing.assert_array_equal(bot, full[..., o[r] + h[r], :])
        assert (sh[r][..., h[r] + 2:, :] == 0).all()
    st = orc.spatial_gather_stacked(sh, Hh, halo=1)
    assert st.shape == (P,) + shape[:-2] + (hmax, shape[-1])
    for r in range(P):
        assert (st[r][..., h[r]:, :] == 0).all()
    np.testing.assert_array_equal(orc.spatial_trim_concat(st, Hh), full)


# ---------------------------------------------------------------------------
# destination-major chunk exchange
# ---------------------------------------------------------------------------
def test_exchange_chunks_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "exchange_chunks_p3_labels.json")))
    table = {}
    x = np.array(_labels_to_codes(g["input"], table), dtype=np.uint16)
    want = np.array(_labels_to_codes(g["output"], table), dtype=np.uint16)
    np.testing.assert_array_equal(orc.exchange_chunks(x), want)


@pytest.mark.parametrize("P,chunk", [(1, 16), (2, 48), (4, 1536), (8, 16)])
def test_exchange_chunks_transpose_and_involution(orc, P, chunk):
    rng = np.random.default_rng(P * chunk)
    x = rng.integers(0, 256, size=(P, P, chunk), dtype=np.uint8)
    y = orc.exchange_chunks(x)
    np.testing.assert_array_equal(y, x.transpose(1, 0, 2))          # library special case
    np.testing.assert_array_equal(orc.exchange_chunks(y), x)         # applied twice: identity


def test_byte_payload_scatter(orc):
    """1-byte payloads (fp8 / int8) move as opaque bytes through the same map."""
    rng = np.random.default_rng(9)
    x = rng.integers(0, 256, size=(4, 2, 5, 8, 16), dtype=np.uint8)
    np.testing.assert_array_equal(orc.scatter(x), _torch_scatter_bytes(x))
    np.testing.assert_array_equal(orc.gather(orc.scatter(x)), x)


def _torch_scatter_bytes(x):
    P, B, S_l, H, D = x.shape
    t = torch.from_numpy(x).view(P, B, S_l, P, H // P, D).permute(3, 1, 0, 2, 4, 5)
    return t.reshape(P, B, P * S_l, H // P, D).contiguous().numpy()
