"""CPU checks of the Python binding's argument checks: every caller-supplied
buffer (out, lse, descales, gradients, workspace) must be a contiguous GPU
tensor on q's device with the exact shape and dtype, checked before any
pointer is taken, since the C ABI receives bare pointers and cannot check
sizes. The tensors here are stand-ins that carry shape, dtype and device
only; taking a pointer from one fails the test."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa


class Fake:
    def __init__(self, shape, dtype=torch.float16, device="cuda:0", contiguous=True):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._contig = contiguous

    def is_contiguous(self):
        return self._contig

    def dim(self):
        return len(self.shape)

    def numel(self):
        return int(np.prod(self.shape))

    def data_ptr(self):
        raise PointerTaken()


class PointerTaken(Exception):
    pass


B, H, S, D = 1, 2, 64, 64
QS = (B, H, S, D)


def qkv(dtype=torch.float16):
    return Fake(QS, dtype), Fake(QS, dtype), Fake(QS, dtype)


GOOD_FWD = dict(out=Fake(QS), lse=Fake((B, H, S), torch.float32), stream=0)

BAD_FWD = {
    "out shape": dict(out=Fake((B, H, S, D + 1))),
    "out on the host": dict(out=Fake(QS, device="cpu")),
    "out on another GPU": dict(out=Fake(QS, device="cuda:1")),
    "out strided": dict(out=Fake(QS, contiguous=False)),
    "out dtype vs o_dtype": dict(out=Fake(QS, torch.float32), o_dtype=torch.float16),
    "out integer": dict(out=Fake(QS, torch.int32)),
    "lse fp16": dict(lse=Fake((B, H, S), torch.float16)),
    "lse shape": dict(lse=Fake((B, H, S + 1), torch.float32)),
    "lse on the host": dict(lse=Fake((B, H, S), torch.float32, device="cpu")),
}


@pytest.mark.parametrize("case", list(BAD_FWD))
def test_fa_fwd_rejects_bad_buffers(case):
    kw = dict(GOOD_FWD)
    kw.update(BAD_FWD[case])
    with pytest.raises(ValueError):
        fa.fa_fwd(*qkv(), **kw)


def test_fa_fwd_good_buffers_reach_the_call():
    with pytest.raises(PointerTaken):
        fa.fa_fwd(*qkv(), **GOOD_FWD)


def test_inputs_on_different_devices():
    q, k, v = qkv()
    k = Fake(QS, device="cuda:1")
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, **GOOD_FWD)


@pytest.mark.parametrize("bad", [
    Fake((2,), torch.float32),                       # two elements
    Fake((1,), torch.float16),                       # not fp32
    Fake((1,), torch.float32, device="cpu"),         # host memory
])
def test_fp8_descales_checked(bad):
    f8 = torch.float8_e4m3fn
    good = Fake((1,), torch.float32)
    for pos in range(3):
        ds = [good, good, good]
        ds[pos] = bad
        with pytest.raises(ValueError):
            fa.fa_fwd(*qkv(f8), descale_q=ds[0], descale_k=ds[1], descale_v=ds[2], **GOOD_FWD)


def test_splitkv_workspace_checked():
    for ws in (Fake((4096,), torch.float32), Fake((4096,), torch.uint8, device="cpu"),
               Fake((64, 64), torch.uint8)):
        with pytest.raises(ValueError):
            fa.fa_fwd_splitkv(*qkv(), num_splits=2, workspace=ws, **GOOD_FWD)


GOOD_BWD_ARGS = lambda: (*qkv(), Fake(QS), Fake(QS), Fake((B, H, S), torch.float32))


@pytest.mark.parametrize("kw", [
    dict(dq=Fake((B, H, S, D + 1))),
    dict(dk=Fake(QS, torch.float32)),                          # dtype differs from dq's
    dict(dv=Fake(QS, device="cuda:1")),
    dict(dq=Fake(QS, contiguous=False)),
    dict(grad_dtype=torch.int8),
    dict(workspace=Fake((1 << 20,), torch.float32)),
    dict(workspace=Fake((1 << 20,), torch.uint8, device="cpu")),
])
def test_fa_bwd_rejects_bad_buffers(kw):
    args = dict(dq=Fake(QS), dk=Fake(QS), dv=Fake(QS), stream=0)
    args.update(kw)
    with pytest.raises(ValueError):
        fa.fa_bwd(*GOOD_BWD_ARGS(), **args)


def test_fa_bwd_lse_and_o_checked():
    q, k, v = qkv()
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, Fake(QS), Fake(QS), Fake((B, H, S), torch.float16), stream=0)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, Fake(QS, device="cuda:1"), Fake(QS), Fake((B, H, S), torch.float32),
                  stream=0)


def test_varlen_buffers_checked():
    q = Fake((100, H, D))
    k = v = Fake((120, H, D))
    cu = Fake((3,), torch.int32)
    for kw in (dict(out=Fake((100, H, D + 1))), dict(lse=Fake((B, H, 100), torch.float32)),
               dict(lse=Fake((H, 100), torch.float16))):
        with pytest.raises(ValueError):
            fa.fa_fwd_varlen(q, k, v, cu, cu, 64, stream=0, **kw)
