"""C-ABI checks that need no GPU: the library loads, exports what include/vq.h declares,
and rejects invalid arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vq.h")
LIB = os.path.join(ROOT, "bit_quantized_linear_vq_amd", "libvq.so")

# The calls below pass a fake device address to entry points that must reject them; on a
# machine with a GPU a validation regression would launch a kernel on it, so the module
# runs only where there is none.
pytestmark = [
    pytest.mark.skipif(not os.path.exists(LIB), reason="libvq.so not built"),
    pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present: fake device addresses must not reach it"),
]

OK, INVALID, SHAPE, UNSUP, HIP = range(5)
F16, BF16, F32 = 0, 1, 2
# A fake, 256-byte aligned address: only ever passed to calls that must fail validation.
FAKE = ctypes.c_void_p(0x10000)
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(vq_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import bit_quantized_linear_vq_amd as vq
    return vq._lib


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12, names
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n
    import bit_quantized_linear_vq_amd as vq
    assert set(names) == set(vq.EXPORTS)


def test_status_strings_and_version(lib):
    for s in range(5):
        assert lib.vq_status_string(s)
    assert b"gfx950" in lib.vq_version()


def test_layout_helpers(lib):
    assert lib.vq_outlier_part_len(0) == 0
    assert lib.vq_outlier_part_len(1) == 64
    assert lib.vq_outlier_part_len(64) == 64
    assert lib.vq_outlier_part_len(65) == 128
    assert lib.vq_packed_k(3072, 30) == 3136
    assert lib.vq_packed_k(1920, 0) == 1920
    # Partial and total column sums, then the result block (13 bytes per column + 32).
    assert lib.vq_detect_workspace_elems(12288, 3072) == (256 + 1) * 3072 + (13 * 3072 + 32 + 7) // 8
    assert lib.vq_detect_workspace_elems(10, 7) == 11 * 7 + (13 * 7 + 32 + 7) // 8
    assert lib.vq_route_workspace_elems(65536) == 1024
    assert lib.vq_detect_workspace_elems(0, 5) == 0


def test_weight_bytes(lib):
    """Packed weight sizes: row-major n * row_bytes; 64-byte K pieces ceil(row_bytes / 64)
    pieces of n * 64 bytes (a 4-bit row of kp % 128 == 64 codes pads its last piece)."""
    KB = 0x100
    assert lib.vq_weight_bytes(5760, 1920, 8) == 5760 * 1920
    assert lib.vq_weight_bytes(5760, 1920, 8 | KB) == 5760 * 1920
    assert lib.vq_weight_bytes(3072, 12288, 4) == 3072 * 6144
    assert lib.vq_weight_bytes(3072, 12288, 4 | KB) == 3072 * 6144
    assert lib.vq_weight_bytes(7, 192, 4) == 7 * 96
    assert lib.vq_weight_bytes(7, 192, 4 | KB) == 2 * 7 * 64
    assert lib.vq_weight_bytes(12288, 3136, 4 | KB) == 25 * 12288 * 64
    for bad in ((0, 64, 8), (4, 0, 8), (4, 100, 8), (4, 64, 6), (4, 64, 6 | KB), (4, 64, 8 | 0x200)):
        assert lib.vq_weight_bytes(*bad) == 0, bad


def quant(lib, **kw):
    a = dict(x=FAKE, dt=BF16, m=64, k=1920, ldx=1920, bits=8, bits_dev=NULL, gran=1, had=0, idx=NULL,
             n_out=0, static=NULL, codes=FAKE, scales=FAKE, stream=NULL)
    a.update(kw)
    return lib.vq_quant_act(a["x"], a["dt"], a["m"], a["k"], a["ldx"], a["bits"], a["bits_dev"], a["gran"],
                            a["had"], a["idx"], a["n_out"], a["static"], a["codes"], a["scales"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(x=NULL), INVALID),
    (dict(codes=NULL), INVALID),
    (dict(scales=NULL), INVALID),
    (dict(dt=F32), INVALID),
    (dict(dt=7), INVALID),
    (dict(m=0), INVALID),
    (dict(m=-5), INVALID),
    (dict(ldx=1000), INVALID),
    (dict(bits=5), UNSUP),
    (dict(bits=3), UNSUP),
    (dict(gran=9), INVALID),
    (dict(gran=2, static=NULL), INVALID),
    (dict(k=1000, ldx=1000), SHAPE),
    (dict(k=1984, ldx=1984, had=128), SHAPE),
    (dict(had=64), UNSUP),
    (dict(had=128, idx=FAKE, n_out=3), UNSUP),
    (dict(idx=NULL, n_out=3), INVALID),
    (dict(idx=FAKE, n_out=129), UNSUP),
    (dict(n_out=-1), INVALID),
    (dict(k=65536, ldx=65536), UNSUP),
    (dict(x=ctypes.c_void_p(0x10008)), SHAPE),
    (dict(ldx=1924), SHAPE),
    (dict(codes=ctypes.c_void_p(0x10004)), SHAPE),
])
def test_quant_act_validation(lib, kw, want):
    assert quant(lib, **kw) == want


def pack(lib, **kw):
    a = dict(w=FAKE, dt=BF16, n=64, k=3072, ldw=3072, bits=4, idx=NULL, n_out=0, had=0, codes=FAKE,
             scales=FAKE, stream=NULL)
    a.update(kw)
    return lib.vq_pack_weights(a["w"], a["dt"], a["n"], a["k"], a["ldw"], a["bits"], a["idx"], a["n_out"],
                               a["had"], a["codes"], a["scales"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(w=NULL), INVALID),
    (dict(bits=6), UNSUP),
    (dict(bits=2), UNSUP),
    (dict(k=100, ldw=100), SHAPE),
    (dict(had=128, idx=FAKE, n_out=4), UNSUP),
    (dict(n=0), INVALID),
    (dict(idx=FAKE, n_out=3072), UNSUP),
    (dict(bits=6 | 0x100), UNSUP),
    (dict(bits=8 | 0x200), UNSUP),
    (dict(bits=4 | 0x100, k=100, ldw=100), SHAPE),  # the layout flag passes to the other checks
    (dict(bits=8 | 0x100, w=NULL), INVALID),
])
def test_pack_weights_validation(lib, kw, want):
    assert pack(lib, **kw) == want


def gemm(lib, **kw):
    a = dict(a=FAKE, sa=FAKE, tok=1, b=FAKE, bb=8, sb=FAKE, m=100, n=64, kp=1920, k0=1920, y=FAKE, odt=BF16,
             ldy=64, acc=NULL, ws=NULL, stream=NULL)
    a.update(kw)
    return lib.vq_qgemm_dequant(a["a"], a["sa"], a["tok"], a["b"], a["bb"], a["sb"], a["m"], a["n"], a["kp"],
                                a["k0"], a["y"], a["odt"], a["ldy"], a["acc"], a["ws"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(a=NULL), INVALID),
    (dict(ws=ctypes.c_void_p(0x10008)), SHAPE),  # workspace not 16-byte aligned
    (dict(sb=NULL), INVALID),
    (dict(y=NULL), INVALID),
    (dict(odt=5), INVALID),
    (dict(tok=2), INVALID),
    (dict(m=0), INVALID),
    (dict(n=-1), INVALID),
    (dict(ldy=32), INVALID),
    (dict(bb=6), UNSUP),
    (dict(kp=1900, k0=1900), SHAPE),
    (dict(k0=1900), SHAPE),
    (dict(k0=2048), SHAPE),
    (dict(kp=3200, k0=3008), SHAPE),  # outlier partition longer than 128
    (dict(y=ctypes.c_void_p(0x10001)), SHAPE),
    (dict(a=ctypes.c_void_p(0x10008)), SHAPE),
    # int32 accumulators: partition 0 no longer than 133120 (int8 weights) or 150976 codes (4-bit)
    (dict(kp=133184, k0=133184), SHAPE),
    (dict(kp=133248, k0=133184), SHAPE),
    (dict(bb=4, kp=151040, k0=151040), SHAPE),
    # the weight layout flag: accepted with both widths, then the same checks
    (dict(bb=6 | 0x100), UNSUP),
    (dict(bb=8 | 0x400), UNSUP),
    (dict(bb=8 | 0x100, kp=133184, k0=133184), SHAPE),
    (dict(bb=4 | 0x100, kp=151040, k0=151040), SHAPE),
    (dict(bb=8 | 0x100, y=ctypes.c_void_p(0x10001)), SHAPE),
    (dict(bb=4 | 0x100, b=NULL), INVALID),
])
def test_qgemm_validation(lib, kw, want):
    assert gemm(lib, **kw) == want


def had(lib, **kw):
    a = dict(x=FAKE, idt=BF16, ldx=256, y=ctypes.c_void_p(0x20000), odt=BF16, ldy=256, rows=4, cols=256,
             block=128, norm=1, stream=NULL)
    a.update(kw)
    return lib.vq_hadamard_block(a["x"], a["idt"], a["ldx"], a["y"], a["odt"], a["ldy"], a["rows"], a["cols"],
                                 a["block"], a["norm"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(x=NULL), INVALID),
    (dict(block=64), UNSUP),
    (dict(cols=192, ldx=192, ldy=192), SHAPE),
    (dict(norm=2), INVALID),
    (dict(idt=4), INVALID),
    (dict(y=FAKE), INVALID),  # in place is not allowed
    (dict(ldx=100), INVALID),
    (dict(ldx=260), SHAPE),
])
def test_hadamard_validation(lib, kw, want):
    assert had(lib, **kw) == want


def test_detect_and_route_validation(lib):
    n_out = ctypes.c_int32(0)
    buf = (ctypes.c_uint8 * 16)()
    idx = (ctypes.c_int32 * 16)()
    assert lib.vq_detect_outliers(NULL, BF16, 8, 16, 16, 3.5, 2.0, 1.0, FAKE, NULL, buf, idx,
                                  ctypes.byref(n_out), NULL, NULL) == INVALID
    assert lib.vq_detect_outliers(FAKE, F32, 8, 16, 16, 3.5, 2.0, 1.0, FAKE, NULL, buf, idx,
                                  ctypes.byref(n_out), NULL, NULL) == INVALID
    assert lib.vq_detect_outliers(FAKE, BF16, 8, 16, 8, 3.5, 2.0, 1.0, FAKE, NULL, buf, idx,
                                  ctypes.byref(n_out), NULL, NULL) == INVALID
    assert lib.vq_detect_outliers(FAKE, BF16, 8, 16, 16, float("nan"), 2.0, 1.0, FAKE, NULL, buf, idx,
                                  ctypes.byref(n_out), NULL, NULL) == INVALID
    assert lib.vq_route_rel_l1(FAKE, FAKE, BF16, 0, 0.1, 8, 4, FAKE, NULL, FAKE, NULL) == INVALID
    assert lib.vq_route_rel_l1(FAKE, FAKE, BF16, 16, 0.1, 5, 4, FAKE, NULL, FAKE, NULL) == INVALID
    assert lib.vq_route_rel_l1(FAKE, FAKE, BF16, 16, 0.1, 8, 4, FAKE, NULL, NULL, NULL) == INVALID


def test_valid_call_without_gpu_reports_hip_error(lib):
    """With no GPU, a call that passes validation must fail cleanly in the HIP runtime."""
    st = quant(lib)
    assert st == HIP
    assert lib.vq_last_hip_error() != 0
    assert gemm(lib) == HIP


def test_decomposition_workspace_size(lib):
    # float32 [2 n_rows x n]: both terms of every listed row.
    assert lib.vq_residual_workspace_bytes(17776, 0, 5760) == 0
    assert lib.vq_residual_workspace_bytes(17776, 889, 5760) == 8 * 889 * 5760
    assert lib.vq_residual_workspace_bytes(10, 3, 7) == 168
    assert lib.vq_residual_workspace_bytes(0, 0, 8) == 0
    assert lib.vq_residual_workspace_bytes(8, 9, 8) == 0  # more rows listed than exist


def resid(lib, **kw):
    a = dict(x=FAKE, dt=BF16, m=64, k=1920, ldx=1920, bits1=8, bits2=8, rows=FAKE, n_rows=4, codes=FAKE,
             scales=FAKE, stream=NULL)
    a.update(kw)
    return lib.vq_quant_residual(a["x"], a["dt"], a["m"], a["k"], a["ldx"], a["bits1"], a["bits2"], a["rows"],
                                 a["n_rows"], a["codes"], a["scales"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(x=NULL), INVALID),
    (dict(rows=NULL), INVALID),
    (dict(codes=NULL), INVALID),
    (dict(scales=NULL), INVALID),
    (dict(dt=F32), INVALID),
    (dict(m=0), INVALID),
    (dict(ldx=1000), INVALID),
    (dict(n_rows=-1), INVALID),
    (dict(n_rows=65), INVALID),
    (dict(bits1=5), UNSUP),
    (dict(bits2=2), UNSUP),
    (dict(k=1000, ldx=1000), SHAPE),
    (dict(ldx=1924), SHAPE),
    (dict(x=ctypes.c_void_p(0x10008)), SHAPE),
    (dict(codes=ctypes.c_void_p(0x10004)), SHAPE),
    (dict(n_rows=0, rows=NULL, codes=NULL, scales=NULL), OK),  # nothing to do, nothing enqueued
])
def test_quant_residual_validation(lib, kw, want):
    assert resid(lib, **kw) == want


def gemm_res(lib, **kw):
    a = dict(a=FAKE, sa=FAKE, b=FAKE, bits=8, sb=FAKE, m=256, n=512, kp=512, a2=FAKE, sa2=FAKE, rows=FAKE,
             n_rows=3, y=FAKE, out=BF16, ldy=512, ws=FAKE, stream=NULL)
    a.update(kw)
    return lib.vq_qgemm_dequant_residual(a["a"], a["sa"], a["b"], a["bits"], a["sb"], a["m"], a["n"], a["kp"],
                                         a["a2"], a["sa2"], a["rows"], a["n_rows"], a["y"], a["out"], a["ldy"],
                                         a["ws"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(n_rows=-1), INVALID),
    (dict(n_rows=257), INVALID),
    (dict(a2=NULL), INVALID),
    (dict(sa2=NULL), INVALID),
    (dict(rows=NULL), INVALID),
    (dict(ws=NULL), INVALID),
    (dict(a=NULL), INVALID),
    (dict(out=9), INVALID),
    (dict(ldy=100), INVALID),
    (dict(bits=6), UNSUP),
    (dict(kp=500), SHAPE),
    (dict(a2=ctypes.c_void_p(0x10004)), SHAPE),
    (dict(ws=ctypes.c_void_p(0x10008)), SHAPE),
    (dict(y=ctypes.c_void_p(0x10001)), SHAPE),
])
def test_qgemm_residual_validation(lib, kw, want):
    assert gemm_res(lib, **kw) == want


MXFP6, MXFP4 = 2, 4


def test_mx_size_helpers(lib):
    assert lib.vq_mx_code_bytes(17776, 12288, MXFP4) == 17776 * 6144
    assert lib.vq_mx_code_bytes(10, 128, MXFP6) == 10 * 96
    assert lib.vq_mx_code_bytes(10, 100, MXFP4) == 0
    assert lib.vq_mx_code_bytes(10, 128, 3) == 0
    # FP4 codes in 64-byte K pieces: ceil(k / 2 / 64) pieces of rows * 64 bytes
    assert lib.vq_mx_code_bytes(3072, 12288, MXFP4 | 0x100) == 96 * 3072 * 64
    assert lib.vq_mx_code_bytes(10, 192, MXFP4 | 0x100) == 2 * 10 * 64
    assert lib.vq_mx_code_bytes(10, 192, MXFP6 | 0x100) == 0
    # step-major E8M0 scales: [k/64][rows rounded up to 8][2]
    assert lib.vq_mx_scale_bytes(17776, 12288) == 192 * 17776 * 2
    assert lib.vq_mx_scale_bytes(3, 128) == 2 * 8 * 2
    assert lib.vq_mx_scale_bytes(0, 128) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(x=NULL), INVALID),
    (dict(codes=NULL), INVALID),
    (dict(scales=NULL), INVALID),
    (dict(dt=F32), INVALID),
    (dict(rows=0), INVALID),
    (dict(ldx=100), INVALID),
    (dict(fmt=3), UNSUP),
    (dict(fmt=MXFP6 | 0x100), UNSUP),  # K pieces hold FP4 codes only
    (dict(fmt=MXFP4 | 0x100, k=96, ldx=96), SHAPE),
    (dict(k=96, ldx=96), SHAPE),
    (dict(ldx=132), SHAPE),
    (dict(x=ctypes.c_void_p(0x10008)), SHAPE),
    (dict(codes=ctypes.c_void_p(0x10004)), SHAPE),
])
def test_mx_quant_validation(lib, kw, want):
    a = dict(x=FAKE, dt=BF16, rows=64, k=128, ldx=128, fmt=MXFP4, codes=FAKE, scales=FAKE, stream=NULL)
    a.update(kw)
    assert lib.vq_mx_quant(a["x"], a["dt"], a["rows"], a["k"], a["ldx"], a["fmt"], a["codes"], a["scales"],
                           a["stream"]) == want


def test_mx_quant_rotated_validation(lib):
    def call(x=FAKE, dt=BF16, rows=64, k=256, ldx=256, fmt=MXFP4, off=0, codes=FAKE, scales=FAKE):
        return lib.vq_mx_quant_rotated(x, dt, rows, k, ldx, fmt, off, codes, scales, NULL)
    assert call(x=NULL) == INVALID
    assert call(dt=F32) == INVALID
    assert call(rows=0) == INVALID
    assert call(ldx=128) == INVALID
    assert call(off=65) == INVALID
    assert call(fmt=3) == UNSUP
    assert call(fmt=MXFP6 | 0x100) == UNSUP
    assert call(fmt=MXFP4 | 0x100, k=192, ldx=192) == SHAPE
    assert call(k=192, ldx=192) == SHAPE  # not a multiple of the 128-point block
    assert call(codes=ctypes.c_void_p(0x10004)) == SHAPE


@pytest.mark.parametrize("kw,want", [
    (dict(a=NULL), INVALID),
    (dict(sb=NULL), INVALID),
    (dict(y=NULL), INVALID),
    (dict(out=5), INVALID),
    (dict(m=0), INVALID),
    (dict(ldy=10), INVALID),
    (dict(fa=3), UNSUP),
    (dict(fb=MXFP6), UNSUP),
    (dict(fa=MXFP4 | 0x100), UNSUP),  # activations are not taken in K pieces
    (dict(fb=MXFP6 | 0x100), UNSUP),
    (dict(fb=MXFP4 | 0x100, k=96), SHAPE),
    (dict(fb=MXFP4 | 0x100, b=ctypes.c_void_p(0x10004)), SHAPE),
    (dict(k=96), SHAPE),
    (dict(sa=ctypes.c_void_p(0x10008)), SHAPE),
    (dict(b=ctypes.c_void_p(0x10004)), SHAPE),
    (dict(y=ctypes.c_void_p(0x10001)), SHAPE),
    (dict(ws=ctypes.c_void_p(0x10008)), SHAPE),
])
def test_mx_gemm_validation(lib, kw, want):
    a = dict(a=FAKE, sa=FAKE, fa=MXFP4, b=FAKE, sb=FAKE, fb=MXFP4, m=64, n=64, k=128, y=FAKE, out=BF16, ldy=64,
             ws=NULL, stream=NULL)
    a.update(kw)
    assert lib.vq_mx_gemm(a["a"], a["sa"], a["fa"], a["b"], a["sb"], a["fb"], a["m"], a["n"], a["k"], a["y"],
                          a["out"], a["ldy"], a["ws"], a["stream"]) == want


def test_mx_gemm_workspace_sizes(lib):
    """Two float32 partials of 256 KB per tile past the last whole round, from 96 steps of 64."""
    part = 256 * 256 * 4
    assert lib.vq_mx_gemm_workspace_bytes(17776, 3072, 12288) == 4096 + 72 * 2 * part
    assert lib.vq_mx_gemm_workspace_bytes(300, 320, 6144) == 4096 + 4 * 2 * part
    assert lib.vq_mx_gemm_workspace_bytes(17776, 5760, 1920) == 0
    assert lib.vq_mx_gemm_workspace_bytes(300, 320, 6100) == 0  # K not a multiple of 64


def test_gemm_tile_count_bound(lib):
    """Output shapes whose 256 x 256 tile count exceeds 2^28 are refused (the kernels
    count tiles in 32 bits), and their workspace size is reported as 0."""
    big = 1 << 30  # 2^22 x 2^22 tiles
    assert lib.vq_qgemm_workspace_bytes(big, big, 6144) == 0
    assert lib.vq_mx_gemm_workspace_bytes(big, big, 6144) == 0
    assert lib.vq_qgemm_dequant(FAKE, FAKE, 1, FAKE, 8, FAKE, big, big, 64, 64, FAKE, BF16, big, NULL, NULL,
                                NULL) == UNSUP
    assert lib.vq_mx_gemm(FAKE, FAKE, MXFP4, FAKE, FAKE, MXFP4, big, big, 64, FAKE, BF16, big, NULL, NULL) == UNSUP
    assert lib.vq_gemm_dense(FAKE, FAKE, BF16, big, big, 64, 64, 64, FAKE, BF16, big, NULL) == UNSUP
    # the largest accepted count: 2^14 x 2^14 tiles
    assert lib.vq_gemm_dense(FAKE, FAKE, BF16, 1 << 22, 1 << 22, 96, 96, 96, FAKE, BF16, 1 << 22, NULL) == SHAPE


def test_gemm_dense_validation(lib):
    def call(x=FAKE, w=FAKE, dt=BF16, m=64, n=64, k=128, ldx=128, ldw=128, y=FAKE, out=BF16, ldy=64):
        return lib.vq_gemm_dense(x, w, dt, m, n, k, ldx, ldw, y, out, ldy, NULL)
    assert call(x=NULL) == INVALID
    assert call(w=NULL) == INVALID
    assert call(y=NULL) == INVALID
    assert call(dt=F32) == INVALID       # inputs are 16-bit
    assert call(out=7) == INVALID
    assert call(m=0) == INVALID
    assert call(ldx=64) == INVALID
    assert call(ldw=96) == INVALID
    assert call(ldy=32) == INVALID
    assert call(k=96, ldx=96, ldw=96) == SHAPE  # K a multiple of 64
    assert call(x=ctypes.c_void_p(0x10008)) == SHAPE
    assert call(ldw=132) == SHAPE         # row pitch not a multiple of 8 elements
    assert call(y=ctypes.c_void_p(0x10001)) == SHAPE


def test_calib_validation(lib):
    assert lib.vq_calib_hist_bins() == 32768
    pct = (ctypes.c_double * 2)(100.0, 99.9)
    bad_pct = (ctypes.c_double * 2)(100.0, 0.0)
    many = (ctypes.c_double * 65)(*([99.0] * 65))

    def call(x=FAKE, dt=BF16, rows=64, cols=128, ldx=128, bits=8, p=pct, n=2, hist=FAKE, out=FAKE):
        # Every call here fails validation, so no device pointer is touched.
        return lib.vq_calib_static_scale(x, dt, rows, cols, ldx, bits, p, n, hist, out, FAKE, FAKE, FAKE,
                                         NULL, NULL)
    assert call(x=NULL) == INVALID
    assert call(hist=NULL) == INVALID
    assert call(out=NULL) == INVALID
    assert call(dt=F32) == INVALID
    assert call(n=0) == INVALID
    assert call(p=many, n=65) == INVALID
    assert call(p=bad_pct) == INVALID
    assert call(ldx=100) == INVALID
    assert call(bits=5) == UNSUP
    assert call(rows=70000, cols=65536, ldx=65536) == UNSUP
    assert call(cols=100, ldx=100) == SHAPE
    assert call(x=ctypes.c_void_p(0x10008)) == SHAPE


def test_step_control_validation(lib):
    import bit_quantized_linear_vq_amd as vq
    assert ctypes.sizeof(vq.ControlParams) == 48 and vq.ControlParams.route_threshold.offset == 32
    assert lib.vq_control_workspace_elems() == 2048
    ok = vq.ControlParams(0.05, 0.15, 3, 8, 4, 0.1, 0.01)

    def call(dn=FAKE, do=FAKE, ddt=BF16, nd=64, x=FAKE, y=FAKE, xdt=BF16, nx=64, nout=NULL, ch=0, p=ok,
             state=FAKE, ws=FAKE, skip=FAKE, bits=FAKE):
        # Every call here fails validation, so no device pointer is touched.
        return lib.vq_step_control(dn, do, ddt, nd, x, y, xdt, nx, nout, ch,
                                   ctypes.byref(p) if p is not None else NULL, state, ws, skip, bits, NULL, NULL,
                                   NULL)
    assert call(p=None) == INVALID
    assert call(state=NULL) == INVALID
    assert call(state=ctypes.c_void_p(0x10004)) == INVALID
    assert call(ws=NULL) == INVALID
    assert call(bits=NULL) == INVALID
    assert call(do=NULL) == INVALID
    assert call(y=NULL) == INVALID
    assert call(nd=0) == INVALID
    assert call(xdt=7) == INVALID
    assert call(nout=FAKE, ch=0) == INVALID
    for bad in (vq.ControlParams(float("nan"), 0.15, 3, 8, 4, 0.1, 0.01), vq.ControlParams(0.05, 0.15, -1, 8, 4, 0.1, 0.01),
                vq.ControlParams(0.05, 0.15, 3, 5, 4, 0.1, 0.01), vq.ControlParams(0.05, 0.15, 3, 8, 4, 0.1, float("nan"))):
        assert call(p=bad) == INVALID


def test_gemm_workspace_sizes(lib):
    """Remainder-split workspace (256 persistent workgroups when no GPU is visible): 4 KB of
    counters plus a 256 KB int32 partial per K range of every tile past the last whole
    round, two ranges per tile, only when K has at least 96 stages of 64 codes."""
    part = 256 * 256 * 4
    assert lib.vq_qgemm_workspace_bytes(17776, 3072, 12288) == 4096 + 72 * 2 * part  # 840 tiles
    assert lib.vq_qgemm_workspace_bytes(300, 320, 6144) == 4096 + 4 * 2 * part         # 4 tiles
    assert lib.vq_qgemm_workspace_bytes(17776, 5760, 1920) == 0   # 30 stages: the split does not pay
    assert lib.vq_qgemm_workspace_bytes(17776, 12288, 3072) == 0  # 48 stages
    assert lib.vq_qgemm_workspace_bytes(35552, 3072, 3072) == 0
    assert lib.vq_qgemm_workspace_bytes(4096, 4096, 12288) == 0   # exactly one round
    assert lib.vq_qgemm_workspace_bytes(512, 33280, 8192) == 4096 + 4 * 2 * part   # 260 tiles: 4 left over
    assert lib.vq_qgemm_workspace_bytes(4864, 6144, 8192) == 0    # 456 tiles: 200 left, no room for two ranges
    assert lib.vq_qgemm_workspace_bytes(0, 64, 12288) == 0
