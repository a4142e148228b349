"""The torch binding checks every tensor's shape, dtype, device and layout
before a pointer reaches the C ABI, which sees bare pointers and sizes and
cannot tell a wrong shape or a host tensor.  Runs on the CPU: each case must
raise before any library call or launch."""

import pytest
import torch

import quantized_base_lora_nf4_amd as qn

N, K, M, R = 128, 256, 8, 4


def _weight(device="cpu", code="nf4", N=N, K=K):
    bits = qn.ops.CODE_BITS[code]
    return qn.NF4Weight(codes=torch.zeros(N * K * bits // 8, dtype=torch.uint8, device=device),
                        q8=torch.zeros(N * K // 64, dtype=torch.uint8, device=device),
                        step=torch.zeros(-(-N * K // 64 // 256), dtype=torch.float32,
                                         device=device),
                        N=N, K=K, code=code)


def _bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("bad", ["X", "A", "B", "Y", "U"])
def test_forward_rejects_a_wrong_shape(bad):
    args = dict(X=_bf(M, K), A=_bf(R, K), B=_bf(N, R), Y=_bf(M, N), U_out=_bf(M, R))
    key = "U_out" if bad == "U" else bad
    t = args[key]
    # A's row count is the rank, so its wrong shape is a wrong K
    args[key] = _bf(t.shape[0], t.shape[1] + 64) if bad in ("X", "A") else _bf(t.shape[0] + 1,
                                                                                  t.shape[1])
    with pytest.raises(ValueError, match=f"{bad} has shape"):
        qn.qlora_linear_fwd(_weight(), args["X"], args["A"], args["B"], 2.0, Y=args["Y"],
                            U_out=args["U_out"])


def test_forward_rejects_a_wrong_dtype():
    with pytest.raises(TypeError, match="X must be bf16"):
        qn.qlora_linear_fwd(_weight(), torch.zeros(M, K), _bf(R, K), _bf(N, R), 2.0)


def test_forward_rejects_host_tensors():
    with pytest.raises(ValueError, match="is on cpu"):
        qn.qlora_linear_fwd(_weight(), _bf(M, K), _bf(R, K), _bf(N, R), 2.0, Y=_bf(M, N))


def test_noalloc_forward_rejects_host_tensors_and_shapes():
    with pytest.raises(ValueError, match="Y has shape"):
        qn.qlora_linear_fwd_noalloc(_weight(), _bf(M, K), _bf(R, K), _bf(N, R), 2.0,
                                    Y=_bf(M, N + 8))
    with pytest.raises(ValueError, match="is on cpu"):
        qn.qlora_linear_fwd_noalloc(_weight(), _bf(M, K), _bf(R, K), _bf(N, R), 2.0, Y=_bf(M, N))


@pytest.mark.parametrize("bad", ["dY", "dX", "dA", "dB"])
def test_backward_rejects_a_wrong_shape(bad):
    out = {"dX": _bf(M, K), "dA": _bf(R, K), "dB": _bf(N, R)}
    dY = _bf(M, N)
    if bad == "dY":
        dY = _bf(M, N + 8)
    else:
        out[bad] = _bf(out[bad].shape[0] + 1, out[bad].shape[1])
    with pytest.raises(ValueError, match=f"{bad} has shape"):
        qn.qlora_linear_bwd(_weight(), _bf(M, K), dY, _bf(R, K), _bf(N, R), 2.0,
                            out=(out["dX"], out["dA"], out["dB"]))


def test_weight_arrays_must_match_the_shape_and_code_width():
    w = _weight()
    w.code = "nf3"  # codes were sized for 4 bits
    with pytest.raises(ValueError, match="code width"):
        qn.qlora_linear_fwd(w, _bf(M, K), _bf(R, K), _bf(N, R), 2.0)
    w = _weight()
    w.q8 = w.q8[:-1]
    with pytest.raises(ValueError, match="q8 / step"):
        qn.qlora_linear_fwd(w, _bf(M, K), _bf(R, K), _bf(N, R), 2.0)


def test_codebook_is_marshalled_from_a_list_and_checked_by_the_library():
    """NF4Weight.levels may be any sequence: the binding copies it into a
    host fp32 array that the struct points to; the library's own check
    refuses values outside the contract (no device is touched)."""
    import ctypes
    from quantized_base_lora_nf4_amd import _lib
    w = qn.NF4Weight(codes=torch.empty(0, dtype=torch.uint8), q8=torch.empty(0, dtype=torch.uint8),
                     step=torch.empty(0), N=8, K=64, code="user2", levels=[-1.0, 0.0, 0.25, 1.0])
    st = w.struct()
    got = (ctypes.c_float * 4).from_address(st.levels)
    assert list(got) == [-1.0, 0.0, 0.25, 1.0]
    assert qn.user_table("user2", [-1.0, 0.0, 0.25, 1.0]) == [-0.5, 0.125, 0.625]
    with pytest.raises(_lib.QloraError):
        qn.user_table("user2", [-1.0, 0.0, 1e-9, 1.0])
    with pytest.raises(ValueError, match="takes 4 values"):
        qn.nf4_quantize(torch.zeros(8, 64), code="user2", levels=[0.0, 1.0, -1.0])
    with pytest.raises(ValueError, match="device tensor"):
        qn.nf4_quantize(torch.zeros(8, 64), code="user2", levels=[0.0, 1.0, -1.0, 0.5])


def test_dequantize_checks_the_weight_and_its_device_before_the_c_abi():
    w = qn.NF4Weight(codes=torch.empty(8 * 64 // 2, dtype=torch.uint8),
                     q8=torch.empty(8, dtype=torch.uint8), step=torch.empty(1), N=8, K=64)
    with pytest.raises(ValueError, match="is on cpu"):
        qn.nf4_dequantize(w)
    w.q8 = torch.empty(7, dtype=torch.uint8)
    with pytest.raises(ValueError, match="q8 / step"):
        qn.nf4_dequantize(w)
