"""The binding rejects mismatched tensors on the host, before any device call
(the kernels trust the sizes that travel with the pointers). CPU tensors are
enough: every case below fails its shape or dtype check first."""
import pytest
import torch

import block_sparse_long_rbs_amd as rbs

S, Hq, Hkv, D, B = 300, 8, 2, 128, 128
NB = -(-S // B)


def qkv(dtype=torch.bfloat16, d_k=D, hkv=Hkv, s_k=S):
    q = torch.zeros((S, Hq, D), dtype=dtype)
    k = torch.zeros((s_k, hkv, d_k), dtype=dtype)
    v = torch.zeros((s_k, hkv, d_k), dtype=dtype)
    return q, k, v


def csr(n_rows):
    return torch.zeros(n_rows + 1, dtype=torch.int32), torch.zeros(8, dtype=torch.int32)


def test_attention_shapes():
    q, k, v = qkv()
    rp, ci = csr(Hkv * NB)
    with pytest.raises(ValueError):
        rbs.blocksparse_attn_fwd(q, *qkv(d_k=64)[1:], B, rp, ci)          # head dim differs
    with pytest.raises(ValueError):
        rbs.blocksparse_attn_fwd(q, *qkv(s_k=S - 1)[1:], B, rp, ci)       # token count differs
    with pytest.raises(ValueError):
        rbs.blocksparse_attn_fwd(q, k, v[:, :1].contiguous(), B, rp, ci)  # v is not k's shape
    with pytest.raises(TypeError):
        rbs.blocksparse_attn_fwd(q, k.float(), v.float(), B, rp, ci)      # dtypes differ
    with pytest.raises(ValueError):
        rbs.blocksparse_attn_fwd(q, k, v, B, *csr(Hkv * NB + 1))          # row_ptr length
    with pytest.raises(ValueError):
        rbs.blocksparse_attn_fwd(q, k, v, B, rp.long(), ci)               # row_ptr dtype
    with pytest.raises(ValueError):
        rbs.blocksparse_attn_fwd(q, k, v, B, rp, ci, out=torch.zeros((S, Hq, D)))  # out dtype
    with pytest.raises(ValueError):                                        # per-head rows: Hq*nb
        rbs.blocksparse_attn_fwd_per_head(q, k, v, B, rp, ci)


def test_fp8_attention_checks():
    q, k, v = qkv()
    rp, ci = csr(Hkv * NB)
    with pytest.raises(TypeError):
        rbs.blocksparse_attn_fwd_fp8(q, k, v, B, rp, ci)                  # bf16, not e4m3
    q8, k8, v8 = (t.to(torch.float8_e4m3fn) for t in (q, k, v))
    with pytest.raises(ValueError):                                        # out must be bf16
        rbs.blocksparse_attn_fwd_fp8(q8, k8, v8, B, rp, ci,
                                     out=torch.zeros((S, Hq, D), dtype=torch.float32))
    with pytest.raises(ValueError):
        rbs.blocksparse_attn_fwd_fp8(q8, k8, v8, B, *csr(Hq * NB))


def test_stats_select_and_block_mask_shapes():
    q, k, v = qkv()
    with pytest.raises(ValueError):
        rbs.rbs_block_stats(q, k[:, :, :64].contiguous(), B)
    f = torch.float32
    cen, rad = torch.zeros((Hkv, NB, D), dtype=f), torch.zeros((Hkv, NB), dtype=f)
    with pytest.raises(ValueError):
        rbs.rbs_select(cen, rad[:, :1].contiguous(), cen, rad, 0.1, 0.1)
    with pytest.raises(ValueError):
        rbs.rbs_select(cen, rad, cen.double(), rad, 0.1, 0.1)
    with pytest.raises(ValueError):
        rbs.block_mask_attn_fwd(q, k, v, [0, 128, S], [0, 0], 5e5,
                                out=torch.zeros((S, Hq, D - 1), dtype=torch.bfloat16))
