"""The tiled transpose (gemm_transpose) against the oracle's transpose, bit for bit, on
the GPU: random bit patterns of 2- and 4-byte elements (NaN patterns included),
whole tiles, ragged edges, single rows and columns, padded leading dimensions,
misaligned pointers (element-wise path), a large matrix, and guard bands around the
output that must stay untouched."""
import numpy as np
import pytest
import torch

import memory_hierarchy_optimisation_amd as mh
import oracle
import synth

pytestmark = pytest.mark.gpu

GUARD = 512
SENT = {2: 0x5A5A, 4: 0x5A5A5A5A}


def _run(rows, cols, E, ld_in=None, ld_out=None, off_in=0, off_out=0, seed=0):
    ld_in = cols if ld_in is None else ld_in
    ld_out = rows if ld_out is None else ld_out
    print(f"[transpose] {rows}x{cols} E={E} ld_in={ld_in} ld_out={ld_out} off={off_in},{off_out}", flush=True)
    x = synth.raw_matrix(rows, ld_in, E, seed=seed)
    dt = x.dtype
    buf_in = torch.empty(off_in + x.numel() + 1, dtype=dt, device="cuda")
    buf_in[off_in:off_in + x.numel()].copy_(x.reshape(-1))
    n_out = cols * ld_out
    buf_out = torch.full((GUARD + off_out + n_out + GUARD,), SENT[E] if E == 2 else SENT[E], dtype=dt, device="cuda")
    mh.gemm_transpose(buf_in[off_in:], buf_out[GUARD + off_out:], rows, cols, ld_in, ld_out, E)
    torch.cuda.synchronize()
    host = buf_out.cpu().numpy()
    sent = np.array([SENT[E]], dtype=host.dtype)[0]
    assert (host[:GUARD + off_out] == sent).all(), "write before out"
    assert (host[GUARD + off_out + n_out:] == sent).all(), "write after out"
    body = host[GUARD + off_out:GUARD + off_out + n_out].reshape(cols, ld_out)
    assert (body[:, rows:] == sent).all(), "write into the padding columns of out"
    want = oracle.transpose(x.numpy(), rows, cols, ld_in, ld_out).reshape(cols, ld_out)
    bad = body[:, :rows] != want[:, :rows]
    assert not bad.any(), f"{int(bad.sum())} elements differ; first at {np.argwhere(bad)[0].tolist()}"


@pytest.mark.parametrize("E", [2, 4])
@pytest.mark.parametrize("rows,cols", [(64, 64), (256, 512), (1000, 777), (1, 300), (300, 1), (257, 129), (63, 65),
                                       (3, 5)])
def test_shapes(rows, cols, E):
    _run(rows, cols, E)


@pytest.mark.parametrize("E", [2, 4])
@pytest.mark.parametrize("ld_in_pad,ld_out_pad,off_in,off_out", [(8, 8, 0, 0), (3, 5, 0, 0), (0, 0, 1, 0), (0, 0, 0, 3),
                                                                (16, 0, 2, 2)])
def test_padding_and_alignment(E, ld_in_pad, ld_out_pad, off_in, off_out):
    rows, cols = 200, 136
    _run(rows, cols, E, ld_in=cols + ld_in_pad, ld_out=rows + ld_out_pad, off_in=off_in, off_out=off_out, seed=3)


@pytest.mark.parametrize("E", [2, 4])
def test_large(E):
    _run(8192, 8192 if E == 2 else 4096, E, seed=5)


def test_degenerate_and_bad_arguments():
    x = torch.zeros(16, dtype=torch.int32, device="cuda")
    mh.gemm_transpose(x, x, 0, 5, 5, 1, 4)          # empty: no-op, pointers not read
    mh.gemm_transpose(x, x, 4, 0, 1, 4, 4)
    with pytest.raises(mh.GemmError, match="elem_bytes"):
        mh.gemm_transpose(x, x, 2, 2, 2, 2, 8)
    with pytest.raises(mh.GemmError, match="ld_in"):
        mh.gemm_transpose(x, x, 2, 4, 3, 2, 4)
    with pytest.raises(mh.GemmError, match="misaligned"):
        mh.gemm_transpose(x.data_ptr() + 2, x, 2, 2, 2, 2, 4)
    with pytest.raises(mh.GemmError, match="negative"):
        mh.gemm_transpose(x, x, -1, 2, 2, 2, 4)
