"""Host-side argument checks of the Python binding: a tensor of the wrong
dtype, shape, stride or device is rejected with ValueError before anything
reaches the C ABI (which sees raw pointers and could not tell).  CPU tensors
stand in for device tensors: the shape and dtype checks run before the
device check, and a call whose tensors are all well formed but on the host
is rejected by the device check."""
import pytest
import torch

import fp8_scaled_matmul_amd as fm


def _u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def _f32(*shape):
    return torch.ones(shape, dtype=torch.float32)


def _mm(**kw):
    args = dict(a=_u8(256, 512), fa=fm.E4M3, scale_a=_f32(1), ga=fm.TENSOR,
                b=_u8(128, 512), fb=fm.E4M3, scale_b=_f32(1), gb=fm.TENSOR)
    args.update(kw)
    return fm.scaled_mm(**args)


def test_scaled_mm_on_host_tensors_rejected():
    with pytest.raises(ValueError, match="CUDA"):
        _mm()


@pytest.mark.parametrize("kw,msg", [
    (dict(a=torch.zeros((256, 512), dtype=torch.bfloat16)), "a must be"),
    (dict(b=_u8(128, 256)), "disagree on k"),
    (dict(a=_u8(512, 256).t()), "unit column stride"),
    (dict(scale_a=_f32(2)), "scale_a"),
    (dict(scale_a=torch.ones(1, dtype=torch.float64)), "scale_a must be torch.float32"),
    (dict(ga=fm.ROW_1x128, gb=fm.BLOCK_128x128), "scale_a"),                    # (1,) scale for 1x128
    (dict(ga=fm.ROW_1x128, gb=fm.BLOCK_128x128, scale_a=_f32(256, 4)), "scale_b"),
    (dict(ga=fm.BLOCK_128x128), "scale_a is TENSOR"),
    (dict(out=torch.empty((256, 128), dtype=torch.float32)), "out must be"),
    (dict(out=torch.empty((256, 127), dtype=torch.bfloat16)), "shape"),
    (dict(workspace=torch.empty(16, dtype=torch.float32)), "workspace"),
])
def test_scaled_mm_rejects(kw, msg):
    with pytest.raises(ValueError, match=msg):
        _mm(**kw)


def test_scaled_mm_block_scales_accepted_up_to_device():
    # well-formed (ROW_1x128, BLOCK_128x128) scales pass every check but the device one
    with pytest.raises(ValueError, match="CUDA"):
        _mm(ga=fm.ROW_1x128, gb=fm.BLOCK_128x128, scale_a=_f32(256, 4), scale_b=_f32(1, 4))


def test_quantize_rejects():
    x = torch.zeros((256, 384), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x must be"):
        fm.quantize(torch.zeros((4, 4), dtype=torch.float16), fm.E4M3)
    with pytest.raises(ValueError, match="scale"):
        fm.quantize(x, fm.E4M3, fm.ROW_1x128, scale=_f32(1))
    with pytest.raises(ValueError, match="scale"):
        fm.quantize(x, fm.E4M3, fm.BLOCK_128x128, scale=_f32(2, 2))
    with pytest.raises(ValueError, match="out must"):
        fm.quantize(x, fm.E4M3, out=_u8(256, 383))
    with pytest.raises(ValueError, match="out_t must"):
        fm.quantize(x, fm.E4M3, want_t=True, out_t=_u8(256, 384))
    with pytest.raises(ValueError, match="want_t"):
        fm.quantize(x, fm.E4M3, out_t=_u8(384, 256))
    with pytest.raises(ValueError, match="GIVEN"):
        fm.quantize(x, fm.E4M3, mode=fm.GIVEN)
    with pytest.raises(ValueError, match="workspace must"):
        fm.quantize(x, fm.E4M3, workspace=torch.empty(64, dtype=torch.float32))
    with pytest.raises(ValueError, match="CUDA"):
        fm.quantize(x, fm.E4M3, fm.BLOCK_128x128, scale=_f32(2, 3), out=_u8(256, 384),
                    want_t=True, out_t=_u8(384, 256))


def test_quantize_delayed_and_requant_reject():
    x = torch.zeros((128, 128), dtype=torch.bfloat16)
    hist = fm.AmaxHistory.__new__(fm.AmaxHistory)
    hist.length = 4
    hist.values = torch.zeros(3, dtype=torch.float32)
    hist.pos = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="history.values"):
        fm.quantize_delayed(x, fm.E4M3, hist)
    cache = fm.WeightCache.__new__(fm.WeightCache)
    cache.rows, cache.cols, cache.fmt, cache.gran = 128, 64, fm.E4M3, fm.TENSOR
    cache.q = _u8(128, 64)
    with pytest.raises(ValueError, match="master"):
        fm.requant_weights([cache], [torch.zeros((64, 128), dtype=torch.bfloat16)])
    with pytest.raises(ValueError, match="one master per cache"):
        fm.requant_weights([cache], [])
    with pytest.raises(ValueError, match="CUDA"):
        fm.requant_weights([cache], [torch.zeros((128, 64), dtype=torch.bfloat16)])
