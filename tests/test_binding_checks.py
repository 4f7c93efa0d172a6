"""Host-side checks of the Python binding (CPU only): argument errors are raised
before any pointer reaches the library, so nothing is launched."""
import pytest

torch = pytest.importorskip("torch")


def _bwd_args(B=1, Hq=4, Hkv=2, N=8, d=64):
    q = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16)
    k = torch.zeros((B, Hkv, N, d), dtype=torch.bfloat16)
    lse = torch.zeros((B, Hq, N), dtype=torch.float32)
    return q, k, k.clone(), q.clone(), lse, q.clone()


@pytest.mark.parametrize("which,shape", [("dq", (1, 4, 7, 64)), ("dk", (1, 2, 7, 64)), ("dk", (1, 4, 8, 64)),
                                         ("dv", (1, 2, 8, 32)), ("dv", (2, 2, 8, 64))])
def test_bwd_rejects_wrong_gradient_shapes_before_launch(which, shape):
    import tiled_online_softmax_fa_amd as fa

    q, k, v, o, lse, dout = _bwd_args()
    bad = torch.zeros(shape, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=f"{which} has shape"):
        fa.bwd(q, k, v, o, lse, dout, **{which: bad})


def test_bwd_shape_errors_precede_device_errors():
    # CPU tensors of the right shapes get past the shape checks and stop at the device check
    import tiled_online_softmax_fa_amd as fa

    q, k, v, o, lse, dout = _bwd_args()
    with pytest.raises(ValueError, match="GPU device"):
        fa.bwd(q, k, v, o, lse, dout, dq=q.clone(), dk=k.clone(), dv=v.clone())
    with pytest.raises(ValueError, match="o/dout/lse"):
        fa.bwd(q, k, v, o, lse[:, :, :-1], dout)
