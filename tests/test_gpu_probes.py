"""The two bandwidth probes read what they are asked to read: a single word
equal to the probes' sink value, placed anywhere in the data, reaches the
sink exactly when the probe reads it (every other word is zero, so the XOR
of a thread's reads is that word)."""
import numpy as np
import pytest
import torch

from paged_kv_cache_395_amd import ops
from tests._gpu import say

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


def _buffer_with_magic(nbytes, word_index):
    a = np.zeros(nbytes // 4, dtype=np.uint32)
    if word_index is not None:
        a[word_index] = MAGIC
    return torch.from_numpy(a.view(np.int32)).cuda()


@pytest.mark.parametrize("word", [0, 5, 12345, (3 << 20) // 4 - 1])
def test_read_probe_reads_every_word(word):
    say(f"[probe] read, magic at word {word}")
    buf = _buffer_with_magic(3 << 20, word)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.probe_read_bandwidth(buf, sink, workgroups=64)
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == MAGIC


@pytest.mark.parametrize("tile_bytes", [4096, 2048])
def test_gather_probe_reads_the_listed_tiles_only(tile_bytes):
    rng = np.random.default_rng(71)
    ntiles = 300
    order = rng.permutation(ntiles).astype(np.int32)
    listed, unlisted = order[:250], order[250:]
    words = tile_bytes // 4
    tiles = torch.from_numpy(np.concatenate([listed, [ntiles + 5, -3]]).astype(np.int32)).cuda()  # two outside
    cases = [(int(listed[0]), 0, True), (int(listed[-1]), words - 1, True), (int(listed[117]), 777 % words, True),
             (int(unlisted[0]), 3, False)]
    for tile, w, read in cases:
        say(f"[probe] gather {tile_bytes} B tiles, magic in tile {tile} word {w}, listed={read}")
        buf = _buffer_with_magic(ntiles * tile_bytes, tile * words + w)
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        ops.probe_gather_bandwidth(buf, tiles, tile_bytes, sink, workgroups=7)
        got = int(sink.cpu().numpy().view(np.uint32)[0])
        assert got == (MAGIC if read else 0), (tile, w, read)
