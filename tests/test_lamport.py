"""Lamport-style exchange, host side: argument validation of the producer and the consumers.
Every call here is invalid and must be rejected before any device access (the pointers are
fake and never dereferenced)."""
import ctypes

import all_reduce_residual_amd as ar

BF16 = ar.DTYPE_BF16


def test_lamport_validation():
    L = ar.lib()
    rbuf, part, out, status = 0x1000000, 0x4000000, 0x5000000, 0x6000000
    res, gam, ro, no = 0x7000000, 0x8000000, 0x9000000, 0xA000000
    W, M, H = 4, 8, 256               # slot = 4096 bytes, a buffer 16 KiB, rbuf = 3 buffers, 48 KiB
    last = rbuf + 2 * 16384 + 3 * 4096          # slot 3 of buffer 2
    # Producer.
    assert L.ar_lamport_push(part, 4, rbuf, W, M, H, BF16, 0, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_lamport_push(part, -1, rbuf, W, M, H, BF16, 0, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_lamport_push(part, 0, rbuf, W, M, H, BF16, -1, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_lamport_push(part, 0, rbuf, 12, M, H, BF16, 0, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_lamport_push(part, 0, rbuf, W, M, 260, BF16, 0, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_lamport_push(rbuf + 4096, 0, rbuf, W, M, H, BF16, 0, None) == ar.AR_ERR_ALIAS
    # The partial may not overlap any of the three buffers, not only this round's.
    assert L.ar_lamport_push(last, 0, rbuf, W, M, H, BF16, 0, None) == ar.AR_ERR_ALIAS
    assert L.ar_lamport_push(part + 2, 0, rbuf, W, M, H, BF16, 0, None) == ar.AR_ERR_MISALIGNED
    assert L.ar_lamport_push(None, 0, rbuf, W, M, H, BF16, 0, None) == ar.AR_ERR_INVALID_ARG
    # Sum consumer.
    assert L.ar_lamport_sum(rbuf, W, M, H, BF16, 0, out, None, 0, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_lamport_sum(rbuf, W, M, H, BF16, -3, out, status, 0, None) == \
        ar.AR_ERR_INVALID_ARG
    assert L.ar_lamport_sum(rbuf, W, M, H, BF16, 0, out, status + 2, 0, None) == \
        ar.AR_ERR_MISALIGNED
    assert L.ar_lamport_sum(rbuf, W, M, H, BF16, 0, rbuf + 8192, status, 0, None) == \
        ar.AR_ERR_ALIAS
    assert L.ar_lamport_sum(rbuf, W, M, H, BF16, 1, last, status, 0, None) == ar.AR_ERR_ALIAS
    assert L.ar_lamport_sum(rbuf, W, M, H, BF16, 0, out, rbuf + 64, 0, None) == ar.AR_ERR_ALIAS
    assert L.ar_lamport_sum(rbuf, W, M, H, BF16, 0, out, last + 64, 0, None) == ar.AR_ERR_ALIAS
    assert L.ar_lamport_sum(rbuf, W, M, H, BF16, 0, out, out + 64, 0, None) == ar.AR_ERR_ALIAS
    assert L.ar_lamport_sum(rbuf + 8, W, M, H, BF16, 0, out, status, 0, None) == \
        ar.AR_ERR_MISALIGNED
    assert L.ar_lamport_sum(rbuf, 3, M, H, BF16, 0, out, status, 0, None) == \
        ar.AR_ERR_UNSUPPORTED
    # Fused consumer.
    args = (rbuf, W, M, H, BF16, 0)
    assert L.ar_lamport_residual_rmsnorm(*args, res, gam, -1.0, ro, no, status, 0, None) == \
        ar.AR_ERR_INVALID_ARG
    assert L.ar_lamport_residual_rmsnorm(rbuf, W, M, H, BF16, -1, res, gam, 1e-6, ro, no, status,
                                         0, None) == ar.AR_ERR_INVALID_ARG
    assert L.ar_lamport_residual_rmsnorm(*args, rbuf + 4096, gam, 1e-6, ro, no, status, 0,
                                         None) == ar.AR_ERR_ALIAS
    assert L.ar_lamport_residual_rmsnorm(*args, res, gam, 1e-6, last, no, status, 0, None) == \
        ar.AR_ERR_ALIAS
    assert L.ar_lamport_residual_rmsnorm(*args, res, gam, 1e-6, ro, ro, status, 0, None) == \
        ar.AR_ERR_ALIAS
    assert L.ar_lamport_residual_rmsnorm(*args, res, gam, 1e-6, ro, no, ro + 16, 0, None) == \
        ar.AR_ERR_ALIAS
    # Row limits of the fused consumer: 8192 vectors (H = 65536 bf16) for W <= 4, 4096 for W >= 8.
    assert L.ar_lamport_residual_rmsnorm(rbuf, W, M, 65544, BF16, 0, res, gam, 1e-6, ro, no,
                                         status, 0, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_lamport_residual_rmsnorm(rbuf, 8, M, 32776, BF16, 0, res, gam, 1e-6, ro, no,
                                         status, 0, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_lamport_residual_rmsnorm(*args, None, gam, 1e-6, ro, no, status, 0, None) == \
        ar.AR_ERR_INVALID_ARG
    # A receive buffer past 2^60 bytes is refused before any size arithmetic wraps: W M H es =
    # 2^60 exactly fits one buffer of slots, but not the three.
    assert L.ar_lamport_arm(rbuf, 64, 1 << 48, 1 << 5, BF16, None) == ar.AR_ERR_UNSUPPORTED
    assert L.ar_lamport_push(part, 0, rbuf, 64, 1 << 48, 1 << 5, BF16, 0, None) == \
        ar.AR_ERR_UNSUPPORTED
    assert L.ar_lamport_arm(rbuf, 64, 1 << 50, 1 << 5, BF16, None) == ar.AR_ERR_UNSUPPORTED
    # Zero rows: nothing to do.
    assert L.ar_lamport_sum(None, W, 0, H, BF16, 0, None, None, 0, None) == ar.AR_OK
    assert L.ar_lamport_arm(None, W, 0, H, BF16, None) == ar.AR_OK


def test_lamport_binding_shapes():
    """The binding wants the receive buffer as [3, W, M, H]."""
    import pytest
    import torch
    with pytest.raises(ValueError):
        ar._check_rbuf(torch.empty((4, 8, 16), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        ar._check_rbuf(torch.empty((2, 4, 8, 16), dtype=torch.bfloat16))
