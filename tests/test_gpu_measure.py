"""The measurement kernels behind the bench's reference rates, checked for
what they read: the plain streaming read folds every 32-bit word of its
buffer, and the gathered tile read folds every word of each listed tile of
both arrays (ids outside the arrays skipped), with XOR; the folds are
compared with numpy on the same bytes, bit for bit."""
import numpy as np
import pytest

from gpu_harness import log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _xor_words(a):
    return int(np.bitwise_xor.reduce(a.view(np.uint32).ravel(), initial=np.uint32(0)))


def test_stream_read_folds_every_word():
    import paged_kv_cache_write_amd as pk
    rng = np.random.default_rng(71)
    host = rng.integers(0, 2**32, size=(5 * 8192) // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    for waves in (0, 1, 3):
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        pk.stream_read(buf, sink, waves=waves)
        torch.cuda.synchronize()
        assert int(sink.cpu().numpy().view(np.uint32)[0]) == _xor_words(host)


@pytest.mark.parametrize("tile_bytes,num_tiles,units", [(4096, 300, 1000), (1024, 64, 7),
                                                        (16384, 40, 85), (2048, 500, 2040)])
def test_tile_read_folds_the_listed_tiles(tile_bytes, num_tiles, units):
    """Units of 0 to 20 tiles (repeats allowed; ids -1 and num_tiles skipped),
    over enough units that the XCD-aware order has empty positions."""
    import paged_kv_cache_write_amd as pk
    rng = np.random.default_rng(tile_bytes + units)
    words = tile_bytes // 4
    a = rng.integers(0, 2**32, size=(num_tiles, words), dtype=np.uint32)
    b = rng.integers(0, 2**32, size=(num_tiles, words), dtype=np.uint32)
    lens = rng.integers(0, 21, size=units)
    lens[0] = 0
    ids = rng.integers(-1, num_tiles + 1, size=int(lens.sum())).astype(np.int32)
    offsets = np.zeros(units + 1, np.int32)
    offsets[1:] = np.cumsum(lens)
    fold = (np.bitwise_xor.reduce(a, axis=1) ^ np.bitwise_xor.reduce(b, axis=1)).astype(np.uint32)
    valid = ids[(ids >= 0) & (ids < num_tiles)]
    want = int(np.bitwise_xor.reduce(fold[valid], initial=np.uint32(0)))
    ad = torch.from_numpy(a.view(np.int32)).cuda()
    bd = torch.from_numpy(b.view(np.int32)).cuda()
    od, idd = torch.from_numpy(offsets).cuda(), torch.from_numpy(ids).cuda()
    log(f"case tile_read tile={tile_bytes} tiles={num_tiles} units={units} listed={ids.size}")
    for _ in range(3):
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        pk.tile_read(ad, bd, tile_bytes, od, idd, sink)
        torch.cuda.synchronize()
        assert int(sink.cpu().numpy().view(np.uint32)[0]) == want
