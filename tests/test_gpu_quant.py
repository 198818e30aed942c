"""The W8A8 mode's per-row e4m3 quantisation on the GPU (gr00t_quantize_e4m3_rows, the
kernel its GEMMs use) against the oracle's, bit for bit: codes are byte results and both
sides decide them from the same bf16 values with fp32 divisions."""
import numpy as np
import pytest

from flow_matching_dit_amd import head as H
from flow_matching_dit_amd import synth
from gpu_util import say
from oracle import gr00t_oracle as O

pytestmark = pytest.mark.gpu


def _bf16_bits_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _check(h, bits):
    import torch
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    q, sc = h.quantize_e4m3_rows(x)
    torch.cuda.synchronize()
    q, sc = q.cpu().numpy(), sc.cpu().numpy()
    ref_q, ref_sc = O.quantize_e4m3_rows_codes(_bf16_bits_to_f32(bits).astype(np.float64))
    bad = np.argwhere(q != ref_q)
    say(f"[quant] rows={bits.shape[0]} cols={bits.shape[1]}: {len(bad)} code mismatches, "
        f"{int(np.sum(sc != ref_sc))} scale mismatches")
    assert np.array_equal(sc.view(np.uint32), ref_sc.view(np.uint32))
    assert len(bad) == 0, [(tuple(i), int(q[tuple(i)]), int(ref_q[tuple(i)])) for i in bad[:5]]


def _head():
    return H.Gr00tHead(synth.TINY, max_batch=1, max_vl_len=8)


@pytest.mark.parametrize("rows,cols", [(1, 8), (37, 1544), (4352, 1536), (64, 6144), (5, 8200)])
def test_random_rows_bit_exact(rows, cols):
    # rows of N(0, 1) values times per-row magnitudes from 1e-6 to 1e4 (subnormal e4m3 codes,
    # saturation-free quotients), with ragged widths: 1544 and 8200 end inside a 512-value step
    rng = np.random.default_rng(rows * 7 + cols)
    mag = 10.0 ** rng.uniform(-6, 4, size=(rows, 1))
    x = (rng.standard_normal((rows, cols)) * mag).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16: any bf16 pattern
    bits[rows // 2, :] = 0  # an all-zero row: scale 1, codes 0
    h = _head()
    try:
        _check(h, bits)
    finally:
        h.close()


def test_every_bf16_value_up_to_448_bit_exact():
    # amax 448 gives scale 1 exactly, so each code is the e4m3 rounding of the bf16 value
    # itself: every finite bf16 magnitude up to 448 (ties between e4m3 neighbours included),
    # with both signs and zero
    pos = np.arange(0, 0x7F80, dtype=np.uint16)
    pos = pos[_bf16_bits_to_f32(pos) <= 448.0]
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    cols = (len(vals) + 7) // 8 * 8
    row = np.zeros(cols, np.uint16)
    row[:len(vals)] = vals
    bits = np.stack([row, row[::-1].copy()])
    h = _head()
    try:
        _check(h, bits)
    finally:
        h.close()
