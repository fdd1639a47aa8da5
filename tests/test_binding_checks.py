"""The Python binding rejects mis-shaped or mistyped tensors before anything
is launched: every caller-supplied output buffer (out, lse, dq, dk, dv) and
every input of the backward is checked against the shapes the kernels will
address.  CPU tensors suffice: each check fires before the device check and
before the library is called."""
import pytest
import torch

import exact_attention_fwd_amd as fa

bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def test_forward_rejects_bad_out_and_lse():
    q, k, v = t(1, 4, 16, 64), t(1, 2, 16, 64), t(1, 2, 16, 64)
    with pytest.raises(ValueError):
        fa.forward(q, k, v, out=t(1, 4, 15, 64))
    with pytest.raises(TypeError):
        fa.forward(q, k, v, out=t(1, 4, 16, 64, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.forward(q, k, v, lse=t(1, 4, 8, dtype=torch.float32))
    with pytest.raises(TypeError):
        fa.forward(q, k, v, lse=t(1, 4, 16))
    with pytest.raises(ValueError):  # key/value heads must divide the query heads
        fa.forward(q, t(1, 3, 16, 64), t(1, 3, 16, 64))
    with pytest.raises(ValueError):
        fa.forward(q, t(1, 0, 16, 64), t(1, 0, 16, 64))
    with pytest.raises(TypeError):
        fa.forward(q, k, t(1, 2, 16, 64, dtype=torch.float32))


def test_backward_rejects_bad_inputs_and_gradients():
    B, H, Hkv, N, d = 1, 4, 2, 16, 64
    q, k, v, o, do = t(B, H, N, d), t(B, Hkv, N, d), t(B, Hkv, N, d), t(B, H, N, d), t(B, H, N, d)
    lse = t(B, H, N, dtype=torch.float32)
    ok = dict(q=q, k=k, v=v, o=o, dout=do, lse=lse)
    bad_inputs = [
        dict(k=t(B, Hkv, N - 1, d), v=t(B, Hkv, N - 1, d)),   # keys shorter than queries
        dict(k=t(B, Hkv, N, 32), v=t(B, Hkv, N, 32)),         # head dim differs
        dict(k=t(B, 3, N, d), v=t(B, 3, N, d)),               # 3 does not divide 4
        dict(v=t(B, Hkv, N + 1, d)),                          # v unlike k
        dict(o=t(B, H, N - 1, d)),
        dict(dout=t(B, H, N, d - 8)),
        dict(lse=t(B, H, N)),                                  # lse must be fp32
        dict(lse=t(B, H, N - 1, dtype=torch.float32)),
    ]
    for bad in bad_inputs:
        with pytest.raises((ValueError, TypeError)):
            fa.backward(**{**ok, **bad})
    with pytest.raises(TypeError):
        fa.backward(**{**ok, "dout": t(B, H, N, d, dtype=torch.float32)})
    for name, buf in (("dq", t(B, H, N - 1, d)), ("dk", t(B, H, N, d)), ("dv", t(B, Hkv, N, d - 1)),
                      ("dq", t(B, H, N, d, dtype=torch.float32))):
        with pytest.raises((ValueError, TypeError)):
            fa.backward(**ok, **{name: buf})


def test_varlen_rejects_bad_buffers():
    cu = torch.tensor([0, 5, 12], dtype=torch.int32)
    q, k, v = t(12, 4, 64), t(12, 2, 64), t(12, 2, 64)
    with pytest.raises(ValueError):
        fa.forward_varlen(q, k, v, cu, 7, out=t(11, 4, 64))
    with pytest.raises(ValueError):
        fa.forward_varlen(q, k, v, cu, 7, lse=t(12, 4, dtype=torch.float32))  # must be [H, total]
    with pytest.raises(ValueError):
        fa.forward_varlen(q, t(12, 3, 64), t(12, 3, 64), cu, 7)
    o, do, lse = t(12, 4, 64), t(12, 4, 64), t(4, 12, dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.backward_varlen(q, k, v, t(12, 4, 32), do, lse, cu, 7)
    with pytest.raises(ValueError):
        fa.backward_varlen(q, t(11, 2, 64), t(11, 2, 64), o, do, lse, cu, 7)
    with pytest.raises(ValueError):
        fa.backward_varlen(q, k, v, o, do, lse, cu, 7, dk=t(12, 4, 64))
    with pytest.raises(ValueError):
        fa.backward_varlen(q, k, v, o, do, lse, cu.to(torch.int64), 7)


def test_decode_and_prefill_reject_bad_buffers():
    S, H, Hkv, d = 2, 8, 2, 64
    q = t(S, H, d)
    pool = t(3, 2, 256, Hkv, d)
    bt = torch.zeros(S, 2, dtype=torch.int32)
    sl = torch.ones(S, dtype=torch.int32)
    with pytest.raises(ValueError):
        fa.decode_paged(q, pool, bt, sl, out=t(S, H, d + 1))
    with pytest.raises(ValueError):
        fa.decode_paged(q, pool, bt, sl, lse=t(S, H + 1, dtype=torch.float32))
    with pytest.raises(TypeError):
        fa.decode_paged(q, pool, bt, sl, lse=t(S, H))
    with pytest.raises(ValueError):
        fa.decode_paged(t(S, H), pool, bt, sl)
    cu = torch.tensor([0, 3, 5], dtype=torch.int32)
    qp = t(5, H, d)
    with pytest.raises(ValueError):
        fa.prefill_paged(qp, pool, bt, sl, cu, 3, out=t(4, H, d))
    with pytest.raises(ValueError):
        fa.prefill_paged(qp, pool, bt, sl, cu, 3, lse=t(5, H, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.prefill_paged(qp, t(3, 2, 256, 3, d), bt, sl, cu, 3)


def test_rope_rejects_bad_buffers():
    q, k, v = t(1, 4, 16, 64), t(1, 2, 16, 64), t(1, 2, 16, 64)
    c, s = t(16, 32, dtype=torch.float32), t(16, 32, dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.forward_rope(q, k, v, c, s, out=t(1, 4, 16, 32))
    with pytest.raises(ValueError):
        fa.forward_rope(q, k, v, c, s, lse=t(1, 4, 15, dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.forward_rope(q, t(1, 2, 15, 64), t(1, 2, 15, 64), c, s)
    with pytest.raises(ValueError):
        fa.forward_rope(q, t(1, 3, 16, 64), t(1, 3, 16, 64), c, s)
    with pytest.raises(ValueError):
        fa.forward_rope(q, k, v, t(16, 31, dtype=torch.float32), s)
