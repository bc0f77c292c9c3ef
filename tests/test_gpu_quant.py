"""GPU parity of the standalone quantizer and the B layout kernels: the bytes
must equal the oracle's bit for bit, with the hardware convert and with the
software encoder."""
import numpy as np
import pytest

import block_scaled_mxfp4_bf16_amd as mx
import oracle
import synthetic as syn
from tests.gpu_util import to_dev_u16_as_bf16, to_dev_u8, torch_cuda

pytestmark = pytest.mark.gpu

MODES = [0, 1]  # hardware convert, software encoder


@pytest.fixture(params=MODES, ids=["hw", "sw"])
def mode(request):
    mx.mxfp4_set_quant_mode(request.param)
    yield request.param
    mx.mxfp4_set_quant_mode(0)


def gpu_quantize(torch, bits, shuffled=False):
    rows, K = bits.shape
    x = to_dev_u16_as_bf16(torch, bits)
    q, s = mx.quantize(x, shuffled_scales=shuffled)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def exhaustive_groups():
    """Groups whose first element (the anchor) fixes the scale byte s and
    whose other 31 elements run over every bf16 magnitude not above the
    anchor, with both signs -- every (element, scale) pair that quantization
    can produce, for every reachable s in [0, 253]."""
    groups = []
    scales = []
    for E in range(2, 256):
        if E == 2:
            anchor = (2 << 7) | 0x40      # 1.5 * 2^-125: largest amax that still gives s = 0
        elif E == 255:
            anchor = 0x7F7F               # largest finite bf16: rounds up to exponent 255, s = 253
        else:
            anchor = (E << 7) | 0x5F      # 1.7421875 * 2^(E-127): keeps exponent E
        mags = np.arange(anchor + 1, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        pad = (-len(vals)) % 31
        vals = np.concatenate([vals, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 31)
        g = np.empty((vals.shape[0], 32), dtype=np.uint16)
        g[:, 0] = anchor
        g[:, 1:] = vals
        groups.append(g)
        scales.append(np.full(vals.shape[0], max(E - 2, 0), dtype=np.uint8))
    g = np.concatenate(groups)
    s = np.concatenate(scales)
    extra = (-g.shape[0]) % 8
    g = np.concatenate([g, np.zeros((extra, 32), dtype=np.uint16)])
    s = np.concatenate([s, np.zeros(extra, dtype=np.uint8)])
    return g.reshape(-1, 256), s.reshape(-1, 8)


def test_quantize_exhaustive_in_contract(mode):
    torch = torch_cuda()
    bits, want_s = exhaustive_groups()
    q_ref, s_ref = oracle.quantize(bits)
    assert np.array_equal(s_ref, want_s)  # the construction hits every scale byte
    q, s = gpu_quantize(torch, bits)
    assert np.array_equal(s, s_ref)
    mism = np.nonzero(q != q_ref)
    assert mism[0].size == 0, "first mismatching bytes: %s" % [
        (int(bits.reshape(-1, 32)[(r * 128 + c) // 16, 2 * ((r * 128 + c) % 16)]), int(q[r, c]), int(q_ref[r, c]))
        for r, c in zip(mism[0][:5], mism[1][:5])]


@pytest.mark.parametrize("name", list(syn.CONFIGS))
def test_quantize_config_a_matches_oracle(mode, name):
    torch = torch_cuda()
    w = syn.CONFIGS[name]
    a = w.a_bits()
    q_ref, s_ref = oracle.quantize(a)
    q, s = gpu_quantize(torch, a)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s, s_ref)


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 96), (17, 64), (255, 160), (257, 512), (64, 7168)])
def test_quantize_shapes_raw_and_shuffled(mode, rows, K):
    torch = torch_cuda()
    a = syn.normal_bf16(rows * 31 + K, 0, (rows, K))
    a[0, :] = 0  # a zero group
    a[-1, :] = 0x8000  # a negative-zero group
    q_ref, s_ref = oracle.quantize(a)
    q, s = gpu_quantize(torch, a)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    q2, s2 = gpu_quantize(torch, a, shuffled=True)
    assert np.array_equal(q2, q_ref)
    assert np.array_equal(s2.reshape(-1), oracle.shuffle_scales(s_ref, rows, K).reshape(-1))


@pytest.mark.parametrize("N,K", [(16, 32), (32, 64), (48, 96), (2112, 7168), (3072, 1536), (288, 512)])
def test_preshuffle_b_matches_oracle(N, K):
    torch = torch_cuda()
    rng = np.random.default_rng(N + K)
    bq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bs = rng.integers(100, 150, size=(N, K // 32), dtype=np.uint8)
    bw, bss = mx.preshuffle_b(to_dev_u8(torch, bq), to_dev_u8(torch, bs))
    torch.cuda.synchronize()
    assert np.array_equal(bw.cpu().numpy(), oracle.preshuffle_b(bq))
    assert np.array_equal(bss.cpu().numpy().reshape(-1), oracle.shuffle_scales(bs, N, K).reshape(-1))


def test_b_prep_on_gpu_equals_oracle_prep():
    """bf16 B -> quantize -> preshuffle, all on the GPU, equals the oracle's."""
    torch = torch_cuda()
    N, K = 2112, 1024
    b = syn.normal_bf16(5, syn.STREAM_B, (N, K))
    q, s = mx.quantize(to_dev_u16_as_bf16(torch, b))
    bw, bs = mx.preshuffle_b(q, s)
    torch.cuda.synchronize()
    qr, sr = oracle.quantize(b)
    assert np.array_equal(bw.cpu().numpy(), oracle.preshuffle_b(qr))
    assert np.array_equal(bs.cpu().numpy().reshape(-1), oracle.shuffle_scales(sr, N, K).reshape(-1))


@pytest.mark.parametrize("N,K", [(16, 32), (32, 64), (48, 96), (288, 512), (2112, 7168), (3072, 1536), (256, 4160)])
def test_prepare_b_equals_oracle_prep_and_two_step_prep(mode, N, K):
    """The one-launch B preparation equals the oracle's quantize + shuffles
    byte for byte (codes, scales and the 127 padding), and equals the
    library's own quantize followed by preshuffle.  Some groups are scaled
    far apart so the scales span the e8m0 range."""
    torch = torch_cuda()
    b = syn.normal_bf16(7 + N + K, syn.STREAM_B, (N, K))
    b = b.copy()
    b[0, :32] = 0  # an all-zero group
    if N > 16 and K >= 96:
        b[17, 64:96] = (b[17, 64:96].astype(np.uint32) + (20 << 7)).astype(np.uint16)  # x 2^20
        b[3, 32:64] = (b[3, 32:64].astype(np.uint32) - (30 << 7)).astype(np.uint16)    # x 2^-30
    x = to_dev_u16_as_bf16(torch, b)
    bw, bs = mx.prepare_b(x)
    q, s = mx.quantize(x)
    bw2, bs2 = mx.preshuffle_b(q, s)
    torch.cuda.synchronize()
    qr, sr = oracle.quantize(b)
    assert np.array_equal(bw.cpu().numpy(), oracle.preshuffle_b(qr))
    assert np.array_equal(bs.cpu().numpy().reshape(-1), oracle.shuffle_scales(sr, N, K).reshape(-1))
    assert np.array_equal(bw.cpu().numpy(), bw2.cpu().numpy())
    assert np.array_equal(bs.cpu().numpy(), bs2.cpu().numpy())


def test_library_loaded_before_torch_uses_torchs_runtime():
    """Loading the library before anything imports torch must still leave
    one HIP runtime in the process (torch's), and calls must work."""
    import subprocess
    import sys
    from tests.conftest import ROOT
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import block_scaled_mxfp4_bf16_amd as mx\n"
        "mx.lib()\n"
        "import torch\n"
        "x = torch.ones((16, 64), dtype=torch.bfloat16, device='cuda')\n"
        "q, s = mx.quantize(x)\n"
        "torch.cuda.synchronize()\n"
        "assert int(q[0, 0]) == 0x66 and int(s[0, 0]) == 125, (int(q[0, 0]), int(s[0, 0]))\n"  # 1.0 / 2^-2 = 4.0: code 6
        "maps = open('/proc/self/maps').read()\n"
        "libs = {l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}\n"
        "assert len(libs) == 1, libs\n"
        "print('ok')\n" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
