"""Hidden and intermediate sizes that are multiples of 8 but not of the 128-wide GEMM
tiles: the forward and backward take the edge-bounded 128x128x32 tiles (partial
column tiles, a partial last reduction step, and partial weight-gradient row and
column tiles). Full tensors against the fp64 oracle, element by element, in bf16 and
the fp32 checking mode, in both gate/up storage orders; the concatenated order must
also match the interleaved run bit for bit where its tiles hold the same values (as in
the Hysen Labs page on SonicMoE, gate/up formats: one layer, two storage orders).

Issue #68 (question 4) asks for a correct backward in [N_recv, K] layout; the shapes
here are those a model may have, e.g. a hidden size of 2880 = 22.5 tiles of 128.
"""
import numpy as np
import pytest

import synth
from _util import TOL, Gpu, assert_close, gateup_to_concat, np64
from test_gpu_expert import oracle_full, run_case

pytestmark = pytest.mark.gpu

# H, I with their residues: every GEMM of the layer gets a partial column tile, and
# (where noted) a reduction length that is not a multiple of 32
SHAPES = {
    # H = 128 + 72 (H % 32 = 8), I = 72: all seven GEMMs ragged in N and K
    "h200_i72": dict(N=500, H=200, I=72, E=5, K=4, seed=41, p_invalid=0.2),
    # the smallest sizes: one 8-wide chunk, reduction shorter than one step
    "h8_i8": dict(N=90, H=8, I=8, E=3, K=2, seed=42, p_invalid=0.1),
    # ragged H only (I a tile multiple), and ragged I only
    "h264_i128": dict(N=300, H=264, I=128, E=4, K=2, seed=43, p_invalid=0.1),
    "h256_i136": dict(N=300, H=256, I=136, E=4, K=2, seed=44, p_invalid=0.1),
    # several full tiles before the partial ones, about 400 rows per expert
    "h456_i200": dict(N=1000, H=456, I=200, E=6, K=3, seed=45, p_invalid=0.2),
}


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_partial_edge_tiles(dtype, shape):
    run_case(synth.case(**SHAPES[shape]), dtype=dtype)


@pytest.mark.parametrize("shape", ["h200_i72", "h8_i8"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_partial_edge_tiles_concat_layout(dtype, shape):
    d = synth.case(**SHAPES[shape])
    print(f"ragged concat case {shape} dtype={dtype}", flush=True)
    m, f, gr = oracle_full(d)
    gi = Gpu(d, dtype=dtype)
    gc = Gpu(d, dtype=dtype, layout=1)
    for g in (gi, gc):
        g.build()
        g.forward()
        g.backward()
    tol = TOL[dtype]
    assert_close(np64(gc.out), f["out"], tol, "out")
    assert_close(np64(gc.h[:m["P"]]), f["h"], tol, "h_save (interleaved)")
    assert_close(np64(gc.dx), gr["dx"], tol, "dx")
    assert_close(np64(gc.dw_up), gateup_to_concat(gr["dw_up"]), tol, "dw_up (concat)")
    assert_close(np64(gc.dw_down), gr["dw_down"], tol, "dw_down")
    assert_close(gc.dtw.cpu().numpy().astype(np.float64), gr["d_topk_weights"], tol, "dtw")
    for a, b in [(gi.out, gc.out), (gi.h, gc.h), (gi.dw_down, gc.dw_down), (gi.dtw, gc.dtw)]:
        assert np.array_equal(np64(a), np64(b))
    assert np.array_equal(gateup_to_concat(np64(gi.dw_up)), np64(gc.dw_up))


def test_partial_edge_tiles_many_rows():
    """About 2700 rows per expert with H = 2880 / 8 = 360 and I = 184: each persistent
    workgroup walks several ragged tiles, the weight gradients reduce over long segments."""
    run_case(synth.case(N=6000, H=360, I=184, E=8, K=4, seed=46, p_invalid=0.1))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_partial_edge_tiles_max_experts(dtype):
    """1024 experts (about 14 rows each) with H = 136 and I = 72: the edge-bounded tiles
    with the largest tile tables and expert ordering, and most weight-gradient tiles
    partial in both directions."""
    run_case(synth.case(N=2000, H=136, I=72, E=1024, K=8, seed=47, p_invalid=0.1), dtype=dtype)
