"""CPU tests: the Python binding refuses wrongly shaped, typed or laid out
buffers with ValueError before any pointer reaches the library (a wrong size
would otherwise become an out-of-bounds GPU write)."""
import pytest
import torch

import ring_attention_step_amd as ra

T, HQ, HKV, D = 64, 4, 2, 128


def _qkv(dtype=torch.bfloat16):
    q = torch.zeros(T, HQ, D, dtype=dtype)
    k = torch.zeros(T, HKV, D, dtype=dtype)
    return q, k, k.clone()


def _fwd(q, k, v, out, lse):
    ra.ring_attn_forward(q, k, v, out, lse, n_blocks=4, layout=0, mask_mode=1, max_ring_passes=4, scale=0.1,
                         prefetch=False, workspace=torch.zeros(16, dtype=torch.uint8))


@pytest.mark.parametrize("out_shape", [(T, HQ, D - 1), (T - 1, HQ, D), (T, HKV, D), (HQ, T, D)])
def test_forward_refuses_wrong_out_shape(out_shape):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="out must be"):
        _fwd(q, k, v, torch.zeros(out_shape, dtype=torch.bfloat16), None)


def test_forward_refuses_out_layout_and_dtype():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="out must be"):
        _fwd(q, k, v, torch.zeros(HQ, T, D, dtype=torch.bfloat16).transpose(0, 1), None)
    with pytest.raises(ValueError, match="out must be float32 or q's dtype"):
        _fwd(q, k, v, torch.zeros(T, HQ, D, dtype=torch.float16), None)


@pytest.mark.parametrize("lse", [torch.zeros(T, HQ), torch.zeros(HQ, T, dtype=torch.float64),
                                 torch.zeros(HQ, T + 1), torch.zeros(T, HQ).t()])
def test_forward_refuses_wrong_lse(lse):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="lse must be"):
        _fwd(q, k, v, torch.zeros(T, HQ, D, dtype=torch.bfloat16), lse)


def test_forward_refuses_mismatched_inputs():
    q, k, v = _qkv()
    out = torch.zeros(T, HQ, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k and v"):
        _fwd(q, k[:32], v[:32], out, None)
    with pytest.raises(ValueError, match="k and v"):
        _fwd(q, k, v[:, :1], out, None)
    with pytest.raises(ValueError, match="multiple"):
        _fwd(q, torch.zeros(T, 3, D, dtype=torch.bfloat16), torch.zeros(T, 3, D, dtype=torch.bfloat16), out, None)
    with pytest.raises(ValueError, match="one dtype"):
        _fwd(q, k.half(), v.half(), out, None)
    with pytest.raises(ValueError, match="unit head_dim stride"):
        _fwd(q.transpose(1, 2).contiguous().transpose(1, 2), k, v, out, None)


def test_forward_with_good_shapes_still_needs_gpu_tensors():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU tensor"):
        _fwd(q, k, v, torch.zeros(T, HQ, D, dtype=torch.bfloat16), torch.zeros(HQ, T))


def test_step_refuses_wrong_state_buffers():
    q, k, v = _qkv(torch.float32)
    B = 16
    O, m, l = torch.zeros(HQ, B, D), torch.zeros(HQ, B), torch.zeros(HQ, B)
    for bad, name in (((torch.zeros(HQ, B, D - 1), m, l), "O"), ((torch.zeros(B, HQ, D), m, l), "O"),
                      ((O, torch.zeros(HQ, B + 1), l), "m"), ((O, m, torch.zeros(HQ, B, dtype=torch.float64)), "l"),
                      ((O, m, torch.zeros(B, HQ).t()), "l")):
        with pytest.raises(ValueError, match="%s must be" % name):
            ra.ring_attn_step(q[:B], k[:B], v[:B], *bad, first_step=True, scale=0.1)


def test_finalize_refuses_wrong_buffers():
    Bq = 16
    O, m, l = torch.zeros(HQ, Bq, D), torch.zeros(HQ, Bq), torch.zeros(HQ, Bq)
    out = torch.zeros(Bq, HQ, D)
    with pytest.raises(ValueError, match="m must be"):
        ra.ring_attn_finalize(O, torch.zeros(HQ, Bq - 1), l, out)
    with pytest.raises(ValueError, match="O must be"):
        ra.ring_attn_finalize(O.double(), m, l, out)
    with pytest.raises(ValueError, match="lse must be"):
        ra.ring_attn_finalize(O, m, l, out, torch.zeros(Bq, HQ))
    with pytest.raises(ValueError, match="out must be"):
        ra.ring_attn_finalize(O, m, l, torch.zeros(HQ, Bq, D))


def test_merge_refuses_wrong_buffers():
    rows = 16
    acc, blk = torch.zeros(rows, HQ, D), torch.zeros(rows, HQ, D)
    lse = torch.zeros(HQ, rows)
    with pytest.raises(ValueError, match="lse_acc must be"):
        ra.ring_attn_merge(acc, lse.double(), blk, lse)
    with pytest.raises(ValueError, match="lse_blk must be"):
        ra.ring_attn_merge(acc, lse, blk, torch.zeros(rows, HQ))
    with pytest.raises(ValueError, match="must match"):
        ra.ring_attn_merge(acc, lse, blk[:, :1].contiguous(), lse)
