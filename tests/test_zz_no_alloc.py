"""qlin_linear_noalloc (staging in the library's fixed scratch) against
qlin_linear (staging passed in), through the C ABI: the same kernels run, so
the outputs must be identical bit for bit.  Two calls in a row per scheme, the
second with a smaller input, then the first again, so that nothing left in the
scratch by one call reaches the next."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import dev, empty, host, torch_mod

pytestmark = pytest.mark.gpu
W8A8, FP8R, FP8B = 0, 1, 2


def Q():
    import quantized_linear_layers_token_amd as q
    return q


def make_call(scheme, seed, M, K, widths):
    x = W.x_bf16(seed, M, K, heavy_tail=True)
    segs = []
    for j, n in enumerate(widths):
        qw = W.w_int8(seed + 10 * j + 1, n, K) if scheme == W8A8 else W.w_e4m3(seed + 10 * j + 1, n, K)
        sw = W.scale_bf16(seed + 10 * j + 2, (n // 128, K // 128) if scheme == FP8B else (n,))
        segs.append((dev(qw), dev(sw)))
    return dev(x), segs


def run(scheme, x, segs, noalloc):
    """-> list of the segments' bf16 outputs (raw bytes), via the raw C ABI."""
    torch = torch_mod()
    q = Q()
    M, K = x.shape
    ys = [empty(torch, (M * qw.shape[0] * 2,), torch.uint8, fill=0xEE) for qw, _ in segs]
    arr = q.segments_array([(qw, sw, y) for (qw, sw), y in zip(segs, ys)])
    st = torch.cuda.current_stream().cuda_stream
    if noalloc:
        r = q.lib().qlin_linear_noalloc(scheme, x.data_ptr(), M, K, arr, len(segs), q.OUT_BF16, st)
    else:
        qx = empty(torch, (M, K), torch.uint8)
        sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32)
        r = q.lib().qlin_linear(scheme, x.data_ptr(), M, K, arr, len(segs), q.OUT_BF16, qx.data_ptr(), sx.data_ptr(),
                                st)
    assert r == q.QLIN_OK, q.status_string(r)
    torch.cuda.synchronize()
    return [host(y) for y in ys]


@pytest.mark.parametrize("scheme", [W8A8, FP8R, FP8B])
def test_noalloc_matches_qlin_linear(scheme):
    # call 1: 40 tokens over three segments (quantizer + tiled GEMM);
    # call 2: 9 tokens, one segment (quantizer + small-M kernel);
    # call 3: call 1 again after the smaller call has overwritten part of the scratch
    first = make_call(scheme, 7100 + scheme, 40, 4096, (256, 128, 384))
    second = make_call(scheme, 7200 + scheme, 9, 1024, (256,))
    print(f"noalloc scheme {scheme}: M=40 K=4096, then M=9 K=1024, then M=40 again", flush=True)
    ref1 = run(scheme, *first, noalloc=False)
    ref2 = run(scheme, *second, noalloc=False)
    got1 = run(scheme, *first, noalloc=True)
    got2 = run(scheme, *second, noalloc=True)
    got3 = run(scheme, *first, noalloc=True)
    for a, b in zip(ref1, got1):
        assert np.array_equal(a, b), "first call differs"
    for a, b in zip(ref2, got2):
        assert np.array_equal(a, b), "second (smaller) call differs"
    for a, b in zip(ref1, got3):
        assert np.array_equal(a, b), "first call repeated differs"


def test_noalloc_one_launch_and_limit():
    # one token: the one-launch path needs no staging at all
    x, segs = make_call(W8A8, 7300, 1, 4096, (512,))
    assert all(np.array_equal(a, b) for a, b in zip(run(W8A8, x, segs, False), run(W8A8, x, segs, True)))
    # past the scratch: refused before any launch
    q = Q()
    torch = torch_mod()
    K = 4096
    M = q.NOALLOC_MAX_CODE_BYTES // K + 1
    xb = empty(torch, (M, K), torch.int16)
    y = empty(torch, (M, 128), torch.int16)
    with pytest.raises(q.QlinError) as e:
        q.qlin_linear_noalloc(W8A8, xb, [(segs[0][0][:128], segs[0][1][:128], y)])
    assert e.value.status == q.QLIN_ERR_TOO_LARGE
