"""gfx950 lane layouts the GEMM kernels rely on, pinned on the GPU with
single-wavefront probes: the transposing LDS reads (ds_read_b64_tr_b16 /
_b8) and the operand / accumulator mappings of each MFMA used, including the
E4M3 decode of every non-NaN FP8 code inside the matrix core."""
import numpy as np
import pytest
import torch

import oracle
from helpers import dev, host, probes
from mixed_precision_dense_tiled_amd import inputs

pytestmark = pytest.mark.gpu


def _stream():
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("bits", [16, 8])
def test_transposing_read_layout(gpu_ok, bits):
    r = np.random.default_rng(bits)
    image = r.integers(0, 256, 4096, dtype=np.uint8)
    offs = (r.integers(0, 4096 // 8, 64) * 8).astype(np.uint32)
    out = torch.zeros(64 * 8, dtype=torch.uint8, device=gpu_ok)
    t_img, t_off = dev(image), dev(offs.view(np.int32))
    assert probes().mpdt_probe_tr(bits, t_img.data_ptr(), t_off.data_ptr(), out.data_ptr(),
                                  _stream()) == 0
    got = host(out).reshape(64, 8)
    exp = np.zeros((64, 8), np.uint8)
    for lane in range(64):
        g, q = lane // 16, lane % 16
        if bits == 16:
            for e in range(4):   # element e of lane q: row e of column q of the 4x16 block
                a = offs[16 * g + 4 * e + q // 4] + 2 * (q % 4)
                exp[lane, 2 * e:2 * e + 2] = image[a:a + 2]
        else:
            for e in range(8):   # byte e of lane q: row e of column q of the 8x16 block
                exp[lane, e] = image[offs[16 * g + 2 * e + q // 8] + q % 8]
    assert np.array_equal(got, exp)


def _run_mfma(kind, A, B, out_dtype):
    D = torch.zeros((32, 32), dtype=out_dtype, device="cuda:0")
    ta, tb = dev(A), dev(B)
    assert probes().mpdt_probe_mfma(kind, ta.data_ptr(), tb.data_ptr(), D.data_ptr(), _stream()) == 0
    return host(D)


@pytest.mark.parametrize("kind,fmt", [(0, "f16"), (1, "bf16")])
def test_mfma16_layout_exact(gpu_ok, kind, fmt):
    r = np.random.default_rng(kind)
    a = r.integers(-8, 9, (32, 16)).astype(np.float32)
    b = r.integers(-8, 9, (16, 32)).astype(np.float32)
    if fmt == "f16":
        A, B = a.astype(np.float16).view(np.uint16), b.astype(np.float16).view(np.uint16)
    else:
        A = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        B = torch.from_numpy(b).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    D = _run_mfma(kind, A, B, torch.float32)
    assert np.array_equal(D, (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float32))


def test_mfma_i8_layout_exact(gpu_ok):
    r = np.random.default_rng(7)
    A = r.integers(-128, 128, (32, 32)).astype(np.int8)
    B = r.integers(-128, 128, (32, 32)).astype(np.int8)
    D = _run_mfma(2, A, B, torch.int32)
    assert np.array_equal(D, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.int32))


def _e4m3(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_mfma_fp8_layout_and_every_code(gpu_ok):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)   # 254 finite codes
    A = np.resize(codes, 32 * 64).reshape(32, 64).copy()
    A[:, ::7] = np.random.default_rng(3).permutation(np.resize(codes, A[:, ::7].size)).reshape(
        A[:, ::7].shape)
    a = _e4m3(A)
    one = np.uint8(0x38)   # 1.0
    for t in range(2):     # B selects column k = j + 32 t of A: D[i][j] = a[i][j + 32 t]
        B = np.zeros((64, 32), np.uint8)
        B[np.arange(32) + 32 * t, np.arange(32)] = one
        D = _run_mfma(3, A, B, torch.float32)
        assert np.array_equal(D.astype(np.float64), a[:, 32 * t:32 * t + 32])
    seen = set(A[:, :].ravel().tolist())
    assert seen == set(codes.tolist())
    # a general product
    r = np.random.default_rng(11)
    B = r.choice(codes, (64, 32)).astype(np.uint8)
    D = _run_mfma(3, A, B, torch.float32)
    b = _e4m3(B)
    ref = a @ b
    S = np.abs(a) @ np.abs(b)
    # The FP8 matrix path sums its 64 exact products with far less than FP32
    # precision (measured up to ~2e-4 * S on codes spanning the whole E4M3
    # range, where FP32 would give ~2^-22 * S).  The GEMM contract is
    # 1e-3 * S per element; one instruction must stay inside it.
    rel = np.abs(D - ref) / S
    print("fp8 MFMA worst |err| / S:", rel.max())
    assert (rel <= 1e-3).all()


def test_mfma_e5m2_every_code(gpu_ok):
    """Every finite E5M2 code through the FP8 instruction with both format
    fields set to E5M2 (identity selector in B), and a general product."""
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8)   # 248 finite codes
    A = np.resize(codes, 32 * 64).reshape(32, 64).copy()
    a = oracle.e5m2_to_f64(A)
    one = np.uint8(0x3C)   # 1.0
    for t in range(2):
        B = np.zeros((64, 32), np.uint8)
        B[np.arange(32) + 32 * t, np.arange(32)] = one
        D = _run_mfma(4, A, B, torch.float32)
        assert np.array_equal(D.astype(np.float64), a[:, 32 * t:32 * t + 32])
    assert set(A.ravel().tolist()) == set(codes.tolist())
    r = np.random.default_rng(12)
    small = codes[(codes & 0x7F) >= 0x30]          # |x| >= 2^-3: products inside FP32's normal range
    A = r.choice(small, (32, 64)).astype(np.uint8)
    B = r.choice(small, (64, 32)).astype(np.uint8)
    a, b = oracle.e5m2_to_f64(A), oracle.e5m2_to_f64(B)
    D = _run_mfma(4, A, B, torch.float32)
    rel = np.abs(D - a @ b) / (np.abs(a) @ np.abs(b))
    print("e5m2 MFMA worst |err| / S:", rel.max())
    assert (rel <= 1e-3).all()


@pytest.mark.parametrize("off,soff", [(0, 0), (2, 0), (6, 0), (14, 0), (1, 0), (7, 0),
                                      (0, 4), (2, 4), (6, 36), (0, 32772), (3, 5)])
def test_unaligned_16_byte_loads(gpu_ok, off, soff):
    """A 16-byte direct-to-LDS buffer load and a plain 16-byte load from an
    address that is only 2-byte (or 1-byte) aligned, through the lane offset
    or the scalar offset, return the bytes at that address: rows of FP16 /
    8-bit operands whose leading dimension is not a multiple of 16 bytes can
    use the same loads."""
    L = probes()
    size = 65536
    src = np.random.default_rng(off + 17 * soff).integers(0, 256, size, dtype=np.uint8)
    t = dev(src)
    out_dma = torch.zeros(1024, dtype=torch.uint8, device=gpu_ok)
    out_ld = torch.zeros(1024, dtype=torch.uint8, device=gpu_ok)
    assert L.mpdt_probe_unaligned(t.data_ptr(), size, off, soff, size, out_dma.data_ptr(),
                                  out_ld.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    want = src[soff + off:soff + off + 1024]
    assert np.array_equal(host(out_ld), want), "plain load"
    assert np.array_equal(host(out_dma), want), "direct-to-LDS load"


def test_buffer_range_check_covers(gpu_ok):
    """Which offsets the raw-buffer range check covers: with the range ending
    512 bytes in, lanes whose lane offset passes it read zero; a scalar offset
    is reported as covered or not (printed; the kernels do not rely on it)."""
    L = probes()
    size = 65536
    src = np.random.default_rng(5).integers(1, 256, size, dtype=np.uint8)
    t = dev(src)
    out_dma = torch.zeros(1024, dtype=torch.uint8, device=gpu_ok)
    out_ld = torch.zeros(1024, dtype=torch.uint8, device=gpu_ok)
    # lane offset only: lanes 32.. start at byte 512 = the range
    assert L.mpdt_probe_unaligned(t.data_ptr(), size, 0, 0, 512, out_dma.data_ptr(), out_ld.data_ptr(),
                                  _stream()) == 0
    torch.cuda.synchronize()
    got = host(out_dma).reshape(64, 16)
    assert np.array_equal(got[:32].ravel(), src[:512]) and not got[32:].any()
    # scalar offset 256 with the same range: covered iff lanes 16..31 read zero
    assert L.mpdt_probe_unaligned(t.data_ptr(), size, 0, 256, 512, out_dma.data_ptr(), out_ld.data_ptr(),
                                  _stream()) == 0
    torch.cuda.synchronize()
    got = host(out_dma).reshape(64, 16)
    print("scalar offset inside the range check:", not got[16:32].any())
    assert np.array_equal(got[:16].ravel(), src[256:512])
    assert not got[32:].any()


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_mfma_peak_probe_runs_and_accumulates(gpu_ok, kind):
    """The MFMA ceiling probe (a measuring stick, not a layout probe), BF16,
    FP8 and INT8: every thread's accumulator sum is finite, the same on a
    second run, and zero for zero operands; the clock stamps advance."""
    L = probes()
    if kind == 0:
        bits = inputs.to_bf16_bits(inputs.normal_f32((2048 * 8,), 11)).view(np.uint8)
    elif kind == 1:
        bits = inputs.fp8_quantize_rows(inputs.normal_f32((64, 512), 11))[0].reshape(-1)
    else:
        bits = inputs.int_uniform((2048 * 16,), 11, -128, 127, np.int8).view(np.uint8)
    data = dev(np.ascontiguousarray(bits))
    out = torch.empty(256 * 256, dtype=torch.float32, device=gpu_ok)
    stamps = torch.zeros(256 * 4, dtype=torch.int64, device=gpu_ok)
    assert L.mpdt_probe_mfma_peak(kind, data.data_ptr(), 2, out.data_ptr(), stamps.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    first = host(out)
    assert np.isfinite(first).all() and np.abs(first).max() > 0
    assert L.mpdt_probe_mfma_peak(kind, data.data_ptr(), 2, out.data_ptr(), stamps.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(host(out), first)
    q = host(stamps).reshape(256, 4)
    assert (q[:, 1] > q[:, 0]).all() and (q[:, 3] >= q[:, 2]).all()
    zero = dev(np.zeros_like(bits))
    assert L.mpdt_probe_mfma_peak(kind, zero.data_ptr(), 2, out.data_ptr(), stamps.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert not host(out).any()
