"""The Python binding refuses wrong-sized, wrongly typed or misplaced buffers
before any pointer reaches the library (the library sees raw pointers and
trusts the sizes it is given; unsloth-zoo issue #850, Suggested fix: fail
loud).  Every check here fires on the host, on CPU tensors, before the
device check and before any library call."""

import pytest
import torch

import bit_weight_quantization_moeq_amd as moeq

E, R, C = 2, 8, 128


def _nf4(E=E, R=R, C=C, fmt=moeq.FMT_NF4):
    return moeq.QWeight.empty(fmt, E, R, C, device="cpu")


def test_qweight_layout_sizes():
    q = _nf4()
    assert [t for _, t, _ in q.layout()] == [(E, R, C // 2), (E, R * C // 64)]
    q.validate_layout()
    dq = _nf4(fmt=moeq.FMT_NF4_DQ)
    assert [t for _, t, _ in dq.layout()] == [(E, R, C // 2), (E, 1), (E, R * C // 64)]
    dq.validate_layout()
    i8 = moeq.QWeight.empty(moeq.FMT_INT8_ROWWISE, E, R, C, device="cpu")
    assert [t for _, t, _ in i8.layout()] == [(E, R, C), (E, R)]
    i8.validate_layout()


@pytest.mark.parametrize("field,bad", [
    ("qdata", torch.empty((E, R, C // 2 - 1), dtype=torch.uint8)),     # one byte short per row
    ("scales", torch.empty((E, R * C // 64 - 1), dtype=torch.float32)),
    ("qdata", torch.empty((E, R, C), dtype=torch.uint8)),              # int8-sized codes for NF4
])
def test_qweight_wrong_size_raises(field, bad):
    q = _nf4()
    setattr(q, field, bad)
    with pytest.raises(ValueError):
        q.validate_layout()


def test_qweight_wrong_dtype_and_layout_raise():
    q = _nf4()
    q.scales = torch.empty(q.scales.shape, dtype=torch.float16)
    with pytest.raises(TypeError):
        q.validate_layout()
    q = _nf4()
    q.qdata = torch.empty((E, C // 2, R), dtype=torch.uint8).transpose(1, 2)   # right size, not contiguous
    with pytest.raises(ValueError):
        q.validate_layout()
    q = _nf4()
    q.scale_codes = torch.empty((E, R * C // 64), dtype=torch.uint8)          # codes on a plain NF4 tensor
    with pytest.raises(ValueError):
        q.validate_layout()
    with pytest.raises(TypeError):                                            # CPU memory, not pinned
        _nf4().validate()


def test_quantize_out_must_describe_the_source():
    w = torch.empty((E, R, C), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moeq.moeq_quantize_nf4(w, out=_nf4(R=R // 2))
    with pytest.raises(ValueError):
        moeq.moeq_quantize_nf4(w, out=moeq.QWeight.empty(moeq.FMT_INT8_ROWWISE, E, R, C, device="cpu"))
    with pytest.raises(ValueError):
        moeq.moeq_quantize_int8_rowwise(w, out=moeq.QWeight.empty(moeq.FMT_INT8_ROWWISE, E, R, C + 8,
                                                                  device="cpu"))
    with pytest.raises(ValueError):
        moeq.moeq_quantize_nf4(w[0])                                           # not [E, rows, cols]
    with pytest.raises(TypeError):                                             # CPU tensors: refused last
        moeq.moeq_quantize_nf4(w, out=_nf4())


def test_dequantize_out_must_match():
    q = _nf4()
    with pytest.raises(ValueError):
        moeq.moeq_dequantize(q, out=torch.empty((E, R, C - 64), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        moeq.moeq_dequantize(q, out=torch.empty((E, R, C), dtype=torch.float32))


def _routed(T=4, K=2, H=C):
    return (torch.empty((T, H), dtype=torch.bfloat16), torch.empty((T, K), dtype=torch.int32),
            torch.empty((T, K), dtype=torch.float32))


def test_forward_buffers_must_match():
    gu, dn = _nf4(R=2 * 64, C=C), _nf4(R=C, C=64)
    x, idx, w = _routed()
    with pytest.raises(ValueError):                                            # out one row short
        moeq.moeq_experts_forward(x, idx, w, gu, dn, out=torch.empty((3, C), dtype=torch.bfloat16))
    with pytest.raises(ValueError):                                            # weights [T, K-1]
        moeq.moeq_experts_forward(x, idx, w[:, :1].contiguous(), gu, dn)
    with pytest.raises(ValueError):                                            # hidden width != H
        moeq.moeq_experts_forward(torch.empty((4, 64), dtype=torch.bfloat16), idx, w, gu, dn)
    bad = _nf4(R=2 * 64, C=C)
    bad.qdata = bad.qdata[:, :-1].contiguous()
    with pytest.raises(ValueError):                                            # packed weights too small
        moeq.moeq_experts_forward(x, idx, w, bad, dn)
    with pytest.raises(TypeError):                                             # int64 indices
        moeq.moeq_experts_forward(x, idx.long(), w, gu, dn)
    with pytest.raises(TypeError):                                             # everything right but on CPU
        moeq.moeq_experts_forward(x, idx, w, gu, dn)


def test_backward_buffers_must_match():
    gu, dn = _nf4(R=2 * 64, C=C), _nf4(R=C, C=64)
    x, idx, w = _routed()
    g = torch.empty_like(x)
    with pytest.raises(ValueError):
        moeq.moeq_experts_backward(x, idx, w, gu, dn, g[:2].contiguous())
    with pytest.raises(ValueError):
        moeq.moeq_experts_backward(x, idx, w, gu, dn, g, grad_weights=torch.empty((4, 3)))
    with pytest.raises(ValueError):
        moeq.moeq_experts_backward(x, idx, w, gu, dn, g, grad_hidden=torch.empty((4, 64), dtype=torch.bfloat16))


def test_router_outputs_must_match():
    x = torch.empty((4, C), dtype=torch.bfloat16)
    gate = torch.empty((8, C), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moeq.moeq_router_topk(x, gate, 2, top_k_index=torch.empty((4, 3), dtype=torch.int32))
    with pytest.raises(ValueError):
        moeq.moeq_router_topk(x, gate, 2, top_k_weights=torch.empty((5, 2), dtype=torch.float32))
    with pytest.raises(ValueError):
        moeq.moeq_router_topk(x, torch.empty((8, 64), dtype=torch.bfloat16), 2)
    with pytest.raises(ValueError):
        moeq.moeq_router_topk(x, gate, 0)


def test_copy_rejects_unpinned_host_memory():
    with pytest.raises(ValueError):
        moeq.moeq_qweight_copy_async(_nf4(), _nf4())


def test_saved_pair_buffers_must_match():
    gu, dn = _nf4(R=2 * 64, C=C), _nf4(R=C, C=64)
    x, idx, w = _routed()
    T, K = idx.shape
    g = torch.empty_like(x)
    with pytest.raises(ValueError):  # one row short of T*K
        moeq.moeq_experts_forward_save(x, idx, w, gu, dn, gu_saved=torch.empty((T * K - 1, 2 * 64)))
    with pytest.raises(ValueError):  # one column short of 2I
        moeq.moeq_experts_backward_saved(idx, w, gu, dn, torch.empty((T * K, 2 * 64 - 1)), g)
    with pytest.raises(ValueError):  # grad_out with fewer tokens than the routing
        moeq.moeq_experts_backward_saved(idx, w, gu, dn, torch.empty((T * K, 2 * 64)), g[:2].contiguous())
    with pytest.raises(TypeError):  # bf16 pre-activations
        moeq.moeq_experts_backward_saved(idx, w, gu, dn, torch.empty((T * K, 2 * 64), dtype=torch.bfloat16), g)
