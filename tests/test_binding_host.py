"""Host-side checks of the binding's argument validation and of the decode
launch geometry (no GPU): a caller-supplied output buffer of the wrong shape
is refused before anything reaches the library, and every 16-row group the
decode grid launches reads inside the prepared weight's padded rows."""

import pytest
import torch

from int8_quantized_matmul_col_amd import binding


def test_out_of_wrong_shape_is_refused_before_the_device_check():
    good = torch.empty((4, 8), dtype=torch.float16)
    with pytest.raises(ValueError, match="shape"):
        binding._check_out(torch.empty((4, 7), dtype=torch.float16), (4, 8), torch.float16, "out")
    with pytest.raises(ValueError, match="shape"):
        binding._check_out(torch.empty((32,), dtype=torch.float16), (4, 8), torch.float16, "out")
    with pytest.raises(TypeError):
        binding._check_out(torch.empty((4, 8), dtype=torch.float32), (4, 8), torch.float16, "out")
    # the right shape on the host still fails: the library takes device memory only
    with pytest.raises(ValueError, match="GPU"):
        binding._check_out(good, (4, 8), torch.float16, "out")


def _decode_rows(N: int):
    """Rows the decode kernel reads for a weight of N output channels: the
    launcher's grid (G groups of 16 rows per workgroup, G = ceil(groups/256)
    capped at 8) and the kernel's clamp of each row to the last padded row."""
    groups = (N + 15) // 16
    G = min(max((groups + 255) // 256, 1), 8)
    grid = (groups + G - 1) // G
    padded = (N + 255) // 256 * 256
    launched = grid * G * 16
    return launched, padded


@pytest.mark.parametrize("N", [1, 16, 8689, 8704, 11008, 22016, 27648, 28672, 65535, 65536])
def test_decode_rows_stay_in_the_padded_weight(N):
    launched, padded = _decode_rows(N)
    # rows n_base + g*16 + ml for every launched group, clamped as the kernel does
    rows = [min(r, padded - 1) for r in range(launched)]
    assert max(rows) < padded
    assert padded * 1 >= N


def test_decode_grid_overruns_without_the_clamp():
    # the shapes the clamp exists for: more groups launched than padded rows hold
    over = [N for N in range(1, 70000) if _decode_rows(N)[0] > _decode_rows(N)[1]]
    assert 8704 in over and len(over) > 1000
