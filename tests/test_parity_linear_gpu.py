"""GPU parity of the fused projection (qlin_linear: bf16 activations in) against
the CPU oracle, for the three schemes, one to four weight segments sharing one
input, the one-launch paths (one token; two tokens streaming the rows; up to
four tokens rounded inside the small-M matrix-core kernel) and the staged path
(quantizer launch + product: more tokens or long K)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import assert_within_tol, dev, e4m3_equal_mod_zero, empty, host, torch_mod

pytestmark = pytest.mark.gpu
BF16, I32, F32 = 0, 1, 2
W8A8, FP8R, FP8B = 0, 1, 2


def Q():
    import quantized_linear_layers_token_amd as q
    return q


def make_segments(scheme, seed, ns, K):
    segs = []
    for i, n in enumerate(ns):
        if scheme == W8A8:
            qw = W.w_int8(seed + 10 * i, n, K)
        else:
            qw = W.w_e4m3(seed + 10 * i, n, K)
        sw = W.scale_bf16(seed + 10 * i + 1, (n // 128, K // 128) if scheme == FP8B else (n,))
        segs.append((qw, sw))
    return segs


def run_linear(scheme, x, segs, out, staged):
    torch = torch_mod()
    M, K = x.shape
    esz = 2 if out == BF16 else 4
    ys = [empty(torch, (M * qw.shape[0] * esz + 64,), torch.uint8, fill=0xFF) for qw, _ in segs]
    dsegs = [(dev(qw), dev(sw), y) for (qw, sw), y in zip(segs, ys)]
    qx = sx = None
    if staged or M > 1:
        qx = empty(torch, (M, K), torch.uint8, fill=0x55)
        sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32, fill=0x55)
    Q().qlin_linear(scheme, dev(x), dsegs, out=out, q_x=qx, s_x=sx)
    res = []
    for (qw, _), y in zip(segs, ys):
        raw = host(y)
        n = qw.shape[0]
        assert (raw[M * n * esz:] == 0xFF).all(), "guard band overwritten"
        body = raw[:M * n * esz]
        res.append(body.view({BF16: np.uint16, I32: np.int32, F32: np.float32}[out]).reshape(M, n))
    return res, (None if qx is None else host(qx)), (None if sx is None else host(sx))


def oracle_quant(scheme, x):
    if scheme == W8A8:
        return O.quant_act_int8(x)
    return O.quant_act_fp8(x, 128 if scheme == FP8B else 0)


def exact(scheme, qx, sx, qw, sw):
    if scheme == W8A8:
        return O.rescale_rowwise(O.contract_int8(qx, qw), sx, sw)
    if scheme == FP8R:
        return O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    return O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw)


CASES = [
    # (M, K, segment widths)
    (1, 128, [128]),
    (1, 4096, [4096, 1024, 1024]),          # q, k, v of one layer
    (1, 4096, [14336, 14336]),              # gate, up
    (1, 14336, [4096]),                     # down
    (1, 12288, [4096]),                     # Qwen3 down
    (1, 9216, [384, 256]),                  # rows past 8 KiB, ragged last KiB slots (long-row form)
    (1, 16384, [256, 128]),                 # the one-launch limit
    (1, 1152, [256, 384, 128, 640]),        # four segments, ragged widths
    (3, 1024, [256, 128]),                  # small-M kernel rounding the tokens itself
    (40, 512, [384]),                       # staged path (tiled GEMM)
    (64, 1024, [384, 128, 640]),            # three segments in one tiled-GEMM launch
    (300, 512, [1024, 256, 256]),           # q, k, v shaped, several token tiles
]


@pytest.mark.parametrize("scheme", [W8A8, FP8R, FP8B])
@pytest.mark.parametrize("M,K,ns", CASES)
def test_linear_matches_oracle(scheme, M, K, ns):
    x = W.x_bf16(7000 + M + K + len(ns), M, K)
    segs = make_segments(scheme, 7100 + K, ns, K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    for staged in ((False, True) if M == 1 else (True,)):
        ys, qx, sx = run_linear(scheme, x, segs, BF16, staged)
        if qx is not None:
            if scheme == W8A8:
                assert np.array_equal(qx.view(np.int8), qx_ref)
            else:
                assert e4m3_equal_mod_zero(qx, qx_ref)
            assert np.array_equal(sx.view(np.uint32), sx_ref.view(np.uint32))
        for (qw, sw), y in zip(segs, ys):
            ye = exact(scheme, qx_ref, sx_ref, qw, sw)
            assert_within_tol(y, ye, f"scheme {scheme} staged {staged}")
            if scheme == W8A8:
                acc = O.contract_int8(qx_ref, qw)
                assert np.array_equal(y, O.epilogue_f32_order(acc, sx_ref, sw))


def test_linear_int8_accumulator_exact():
    x = W.x_bf16(7300, 1, 4096)
    segs = make_segments(W8A8, 7301, [4096, 1024, 1024], 4096)
    qx_ref, _ = O.quant_act_int8(x)
    ys, _, _ = run_linear(W8A8, x, segs, I32, False)
    for (qw, _), y in zip(segs, ys):
        assert np.array_equal(y, O.contract_int8(qx_ref, qw))


def test_linear_zero_row_and_empty_segment():
    torch = torch_mod()
    x = np.zeros((1, 256), np.uint16)
    qw = W.w_int8(7400, 64, 256)
    sw = W.scale_bf16(7401, 64)
    y = empty(torch, (1, 64), torch.int16, fill=0x7F)
    empty_w = torch.empty((0, 256), dtype=torch.int8, device="cuda")
    Q().qlin_linear(W8A8, dev(x), [(dev(qw), dev(sw), y), (empty_w, None, None)])
    assert not host(y).any()                 # all-zero token -> s = 0 -> y = 0


def test_linear_long_k_uses_staging():
    # K above the one-launch limit at M = 1: q_x / s_x are required staging
    torch = torch_mod()
    K = 16400
    x = W.x_bf16(7500, 1, K)
    qw = W.w_int8(7501, 40, K)
    sw = W.scale_bf16(7502, 40)
    y = empty(torch, (1, 40), torch.int16)
    with pytest.raises(Q().QlinError):
        Q().qlin_linear(W8A8, dev(x), [(dev(qw), dev(sw), y)])
    ys, qx, sx = run_linear(W8A8, x, [(qw, sw)], BF16, True)
    qx_ref, sx_ref = O.quant_act_int8(x)
    assert np.array_equal(qx.view(np.int8), qx_ref)
    assert np.array_equal(ys[0], O.epilogue_f32_order(O.contract_int8(qx_ref, qw), sx_ref, sw))


@pytest.mark.parametrize("scheme", [W8A8, FP8R])
def test_linear_ragged_segments_tiled(scheme):
    # segment widths that are not multiples of any tile edge: every weight
    # panel stays inside its segment, every output row lands in its own buffer
    M, K, ns = 100, 528, [200, 72, 300, 1]
    x = W.x_bf16(7600, M, K)
    segs = make_segments(scheme, 7610, ns, K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    ys, _, _ = run_linear(scheme, x, segs, F32 if scheme == FP8R else I32, True)
    for (qw, sw), y in zip(segs, ys):
        if scheme == W8A8:
            assert np.array_equal(y, O.contract_int8(qx_ref, qw))
        else:
            ye = exact(scheme, qx_ref, sx_ref, qw, sw)
            assert np.max(np.abs(y - ye)) <= 4e-3 * np.max(np.abs(ye))


def one_launch(scheme, M, K, rows):
    """Whether qlin_linear runs as one launch (staging buffers optional):
    one token with K <= 16 Ki; two tokens streaming the rows (K <= 16 Ki, at
    most 64 MiB of weights, block FP8 rows up to 8 KiB); up to four tokens of
    up to 4096 inputs rounded inside the small-M kernel."""
    if M == 1:
        return K <= 16384
    if M == 2 and K <= 16384 and rows * K <= 64 << 20 and not (scheme == FP8B and K > 8192):
        return True
    return M <= 4 and K <= 4096


# two to four tokens: one launch (the staging buffers are optional there)
TOKEN_CASES = [
    # (M, K, segment widths)
    (2, 128, [128]),
    (2, 16384, [128, 256]),              # longest rows
    (2, 1152, [256, 384, 128, 640]),     # four segments, K not a multiple of 1 KiB
    (2, 4096, [4096, 1024, 1024]),       # q, k, v
    (2, 14336, [512]),                   # down-shaped rows
    (3, 128, [128]),
    (3, 4080, [200, 56]),                # K not a multiple of the 128-byte step
    (3, 4112, [200, 56]),                # just past the rows rounded in the kernel: staged
    (4, 1152, [256, 384, 128, 640]),
    (4, 4096, [4096, 1024, 1024]),       # q, k, v
    (4, 12288, [256]),                   # Qwen3 down-shaped rows: staged
    (4, 14336, [384]),                   # Llama down-shaped rows: staged
]


@pytest.mark.parametrize("scheme", [W8A8, FP8R, FP8B])
@pytest.mark.parametrize("M,K,ns", TOKEN_CASES)
def test_linear_few_tokens_one_launch(scheme, M, K, ns):
    if scheme == FP8B and (K % 128 or any(n % 128 for n in ns)):
        pytest.skip("block scheme needs K and N multiples of 128")
    print(f"few tokens scheme {scheme} M={M} K={K} ns={ns}", flush=True)
    x = W.x_bf16(7700 + M + K, M, K)
    if M > 2:
        x[1, : K // 2] = 0                  # a token (or its first groups) all zero
    segs = make_segments(scheme, 7710 + K + M, ns, K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    one = one_launch(scheme, M, K, sum(ns))
    if not one:
        with pytest.raises(Q().QlinError):
            run_linear_opt(scheme, x, segs, BF16, False)
    for staged in ((False, True) if one else (True,)):
        ys, qx, sx = run_linear_opt(scheme, x, segs, BF16, staged)
        if staged:
            if scheme == W8A8:
                assert np.array_equal(qx.view(np.int8), qx_ref)
            else:
                assert e4m3_equal_mod_zero(qx, qx_ref)
            assert np.array_equal(sx.reshape(sx_ref.shape).view(np.uint32), sx_ref.view(np.uint32))
        for (qw, sw), y in zip(segs, ys):
            ye = exact(scheme, qx_ref, sx_ref, qw, sw)
            assert_within_tol(y, ye, f"{M} tokens scheme {scheme} staged {staged}")
            if scheme == W8A8:
                assert np.array_equal(y, O.epilogue_f32_order(O.contract_int8(qx_ref, qw), sx_ref, sw))


def test_linear_few_tokens_ragged_rows_exact():
    # ragged widths and the int32 accumulator of every row, two to four tokens
    for M in (2, 3, 4):
        K = 1040
        x = W.x_bf16(7800 + M, M, K)
        segs = make_segments(W8A8, 7810 + M, [200, 72, 1, 33], K)
        qx_ref, _ = O.quant_act_int8(x)
        ys, _, _ = run_linear_opt(W8A8, x, segs, I32, False)
        for (qw, _), y in zip(segs, ys):
            assert np.array_equal(y, O.contract_int8(qx_ref, qw))


def run_linear_opt(scheme, x, segs, out, staged):
    """qlin_linear with staging buffers only when asked for."""
    torch = torch_mod()
    M, K = x.shape
    esz = 2 if out == BF16 else 4
    ys = [empty(torch, (M * qw.shape[0] * esz + 64,), torch.uint8, fill=0xFF) for qw, _ in segs]
    qx = sx = None
    if staged:
        qx = empty(torch, (M, K), torch.uint8, fill=0x55)
        sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32, fill=0x55)
    Q().qlin_linear(scheme, dev(x), [(dev(qw), dev(sw), y) for (qw, sw), y in zip(segs, ys)], out=out, q_x=qx, s_x=sx)
    res = []
    for (qw, _), y in zip(segs, ys):
        raw = host(y)
        n = qw.shape[0]
        assert (raw[M * n * esz:] == 0xFF).all(), "guard band overwritten"
        res.append(raw[:M * n * esz].view({BF16: np.uint16, I32: np.int32, F32: np.float32}[out]).reshape(M, n))
    return res, (None if qx is None else host(qx)), (None if sx is None else host(sx))


def test_linear_two_tokens_large_call_one_launch():
    # more than 64 MiB of weights at two tokens (the gate/up pair): the small-M
    # kernel rounds the tokens itself, so the staging buffers stay optional
    M, K, ns = 2, 4096, [14336, 14336]
    x = W.x_bf16(7900, M, K)
    segs = make_segments(W8A8, 7910, ns, K)
    qx_ref, sx_ref = O.quant_act_int8(x)
    for staged in (False, True):
        ys, qx, _ = run_linear_opt(W8A8, x, segs, BF16, staged)
        if staged:
            assert np.array_equal(qx.view(np.int8), qx_ref)
        for (qw, sw), y in zip(segs, ys):
            assert np.array_equal(y, O.epilogue_f32_order(O.contract_int8(qx_ref, qw), sx_ref, sw))


def test_linear_five_tokens_need_staging():
    M, K = 5, 1024
    x = W.x_bf16(7950, M, K)
    segs = make_segments(W8A8, 7960, [256], K)
    with pytest.raises(Q().QlinError):
        run_linear_opt(W8A8, x, segs, BF16, False)


@pytest.mark.parametrize("scheme", [FP8R, FP8B])
@pytest.mark.parametrize("M", [2, 3, 4])
def test_linear_few_tokens_f32_out(scheme, M):
    # f32 outputs of the one-launch forms (scales taken from the kernel's own rounding)
    K, ns = 1024, [256, 128]
    x = W.x_bf16(8050 + M, M, K)
    segs = make_segments(scheme, 8060 + M, ns, K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    ys, _, _ = run_linear_opt(scheme, x, segs, F32, False)
    for (qw, sw), y in zip(segs, ys):
        ye = exact(scheme, qx_ref, sx_ref, qw, sw)
        assert np.max(np.abs(y - ye)) <= 4e-3 * np.max(np.abs(ye)), f"f32, scheme {scheme}, M={M}"


def test_readme_example():
    """The Python example of the README, run as written (torch tensors in,
    staging buffers given), checked against the oracle."""
    torch = torch_mod()
    import quantized_linear_layers_token_amd as Qm
    torch.manual_seed(0)
    x = torch.randn(16, 4096, dtype=torch.bfloat16, device="cuda")
    qw = torch.randint(-127, 128, (4096, 4096), dtype=torch.int8, device="cuda")
    sw = (torch.rand(4096, device="cuda") * 4e-3 + 1e-3).to(torch.bfloat16)
    y = torch.empty(16, 4096, dtype=torch.bfloat16, device="cuda")
    qx = torch.empty(16, 4096, dtype=torch.int8, device="cuda")
    sx = torch.empty(16, dtype=torch.float32, device="cuda")
    Qm.qlin_linear(Qm.SCHEME_W8A8, x, [(qw, sw, y)], q_x=qx, s_x=sx)
    torch.cuda.synchronize()

    def bits(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    qx_ref, sx_ref = O.quant_act_int8(bits(x))
    assert np.array_equal(host(qx), qx_ref)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))
    acc = O.contract_int8(qx_ref, host(qw))
    assert np.array_equal(bits(y), O.epilogue_f32_order(acc, sx_ref, bits(sw)))
    assert_within_tol(bits(y), exact(W8A8, qx_ref, sx_ref, host(qw), bits(sw)), "README example")
