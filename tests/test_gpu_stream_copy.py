"""GPU check of osm_stream_copy, the bandwidth-ceiling probe of bench.py.

The copy must reproduce its source byte for byte, for whole 64 KiB chunks,
ragged vector counts and a ragged byte tail, and write nothing outside the
destination range.
"""

import pytest
import torch

import online_softmax_06_amd as osm

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    osm.load_library()


@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 7, 65536, 65536 * 3 + 16 * 5 + 9, 1 << 24])
def test_copy_is_exact_and_stays_in_bounds(nbytes):
    print("[case] osm_stream_copy", nbytes, flush=True)
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    pad = 4096
    buf = torch.full((nbytes + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = buf[pad:pad + nbytes]
    assert src.data_ptr() % 16 == 0 and dst.data_ptr() % 16 == 0
    st = osm.osm_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                             torch.cuda.current_stream().cuda_stream)
    assert st == osm.OSM_OK, osm.osm_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert (buf[:pad] == 0xA5).all() and (buf[pad + nbytes:] == 0xA5).all()
