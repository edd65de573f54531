"""The C-ABI library loads on a machine without a GPU, exports every entry
point declared in include/fp8blk.h, and rejects bad arguments on the host
before any HIP call (so these tests make no GPU call at all).

The pointers passed here are never dereferenced: every call fails validation.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8blk.h")
LIB = os.path.join(ROOT, "fp8_quantization_block_amd", "libfp8blk.so")

OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP = 0, 1, 2, 3, 4
BF16, F32 = 0, 1
PER_TENSOR, GROUP, BLOCK = 0, 1, 2
E4M3, E5M2 = 0, 1

# fake, aligned, never-dereferenced device addresses
PA, PB, PC, PD = 0x10000000, 0x20000000, 0x30000000, 0x40000000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libfp8blk.so not built (python -m fp8_quantization_block_amd.build)")
    import fp8_quantization_block_amd as fp8
    return fp8.load_library(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fp8_quantize", "fp8_block_gemm", "fp8_block_gemm_quant", "fp8_kv_quantize", "fp8_kv_dequantize",
              "fp8_kv_decode_attention", "fp8_kv_decode_attention_workspace_size", "fp8_quantize_mx", "fp8_mx_gemm",
              "fp8_quantize_static", "fp8_scale_from_amax_history", "fp8_kv_decode_attention_noalloc",
              "fp8_quantize_gemm_decode",
              "fp8blk_status_string", "fp8blk_last_error", "fp8blk_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_version_and_strings(lib):
    assert lib.fp8blk_abi_version() == 1
    assert lib.fp8blk_status_string(EALIGN) == b"FP8BLK_EALIGN"
    assert lib.fp8blk_status_string(99) == b"FP8BLK_UNKNOWN"


def q(lib, x=PA, dt=BF16, rows=4, cols=256, ldx=256, gran=GROUP, fmt=E4M3, qp=PB, ldq=256,
      s=PC, ssr=2, ssc=1):
    return lib.fp8_quantize(x, dt, rows, cols, ldx, gran, fmt, qp, ldq, s, ssr, ssc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), EINVAL),
    (dict(qp=0), EINVAL),
    (dict(s=0), EINVAL),
    (dict(rows=-1), EINVAL),
    (dict(cols=-5), EINVAL),
    (dict(ldx=100), EINVAL),
    (dict(ldq=128), EINVAL),
    (dict(dt=7), EINVAL),
    (dict(gran=9), EINVAL),
    (dict(fmt=5), EINVAL),
    (dict(fmt=2), EINVAL),
    (dict(fmt=E5M2, ldx=100), EINVAL),     # E5M2 passes the format check
    (dict(x=PA + 2), EALIGN),
    (dict(qp=PB + 8), EALIGN),
    (dict(ldx=260, cols=256), EALIGN),
    (dict(ldq=264, cols=256), EALIGN),
    (dict(ssr=-1), EINVAL),
    (dict(qp=PA + 256), EINVAL),           # q overlaps x
    (dict(s=PB + 16), EINVAL),             # scales overlap q
    (dict(ssr=0, ssc=1), EINVAL),          # grid rows collapse onto one float
    (dict(ssr=1, ssc=1), EINVAL),          # cells (i, j + 1) and (i + 1, j) share a float
    (dict(s=PC + 2), EALIGN),              # scales not 4-byte aligned
    (dict(ssr=1 << 40), EUNSUPPORTED),
    (dict(rows=1 << 31), EUNSUPPORTED),
])
def test_quantize_rejects(lib, kw, status):
    assert q(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_quantize")


def test_quantize_empty_group_grid_is_a_noop(lib):
    # no HIP call is made for an empty 1x128 or 128x128 grid
    assert q(lib, rows=0) == OK
    assert q(lib, cols=0, gran=BLOCK) == OK
    assert lib.fp8blk_last_error() == b""


def g(lib, M=256, N=256, K=256, a=PA, lda=256, sa=PB, ga=GROUP, sam=2, sak=1, b=PC, ldb=256,
      sb=PB + 65536, gb=BLOCK, sbn=2, sbk=1, fa=E4M3, fb=E4M3, c=PD, cdt=BF16, ldc=256):
    return lib.fp8_block_gemm(M, N, K, a, lda, sa, ga, sam, sak, b, ldb, sb, gb, sbn, sbk, fa, fb,
                              c, cdt, ldc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=0), EINVAL),
    (dict(sb=0), EINVAL),
    (dict(c=0), EINVAL),
    (dict(ga=BLOCK), EINVAL),
    (dict(gb=GROUP), EINVAL),
    (dict(cdt=3), EINVAL),
    (dict(fa=2), EINVAL),
    (dict(fa=E5M2, fb=E5M2, lda=128), EINVAL),   # E5M2 operands pass the format check
    (dict(fb=4), EINVAL),
    (dict(M=-1), EINVAL),
    (dict(N=0), EINVAL),
    (dict(N=200), EUNSUPPORTED),
    (dict(K=200, lda=256, ldb=256), EUNSUPPORTED),
    (dict(lda=128), EINVAL),
    (dict(ldc=128), EINVAL),
    (dict(a=PA + 4), EALIGN),
    (dict(lda=264), EALIGN),
    (dict(ldc=260), EALIGN),
    (dict(c=PA + 1024), EINVAL),           # c overlaps a
    (dict(sak=-2), EINVAL),
    (dict(sa=PB + 2), EALIGN),             # scale arrays not 4-byte aligned
    (dict(sb=PB + 65536 + 1), EALIGN),
    (dict(sbk=1 << 40), EUNSUPPORTED),
    # scale grids spanning 4 GiB or more (the prefill kernel addresses a grid
    # with 32-bit byte offsets): a padded weight grid, a padded activation grid
    (dict(sbn=1 << 30), EUNSUPPORTED),
    (dict(sam=1 << 23), EUNSUPPORTED),
    (dict(ga=PER_TENSOR, sam=1 << 22, c=PA + 1024), EINVAL),   # per tensor ignores the strides (then: c overlaps a)
])
def test_gemm_rejects(lib, kw, status):
    assert g(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_block_gemm")


def gq(lib, M=256, N=256, K=256, a=PA, lda=256, sa=PB, ga=GROUP, sam=2, sak=1, b=PC, ldb=256,
       sb=PB + 65536, gb=BLOCK, sbn=2, sbk=1, fa=E4M3, fb=E4M3, fc=E4M3, qc=PD, ldqc=256,
       sc=PD + (1 << 20), scm=1, scn=256):
    return lib.fp8_block_gemm_quant(M, N, K, a, lda, sa, ga, sam, sak, b, ldb, sb, gb, sbn, sbk, fa, fb, fc,
                                    qc, ldqc, sc, scm, scn, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=0), EINVAL),
    (dict(qc=0), EINVAL),
    (dict(sc=0), EINVAL),
    (dict(fc=2), EINVAL),
    (dict(fc=E5M2, ldqc=128), EINVAL),       # E5M2 output passes the format check
    (dict(N=200), EUNSUPPORTED),
    (dict(qc=PD + 4), EALIGN),
    (dict(ldqc=264), EALIGN),
    (dict(scm=-1), EINVAL),
    (dict(scm=0), EINVAL),                   # rows collapse onto one scale
    (dict(scn=0), EINVAL),                   # groups collapse onto one scale
    (dict(qc=PA + 1024), EINVAL),            # codes overlap a
    (dict(sc=PD + 4096), EINVAL),            # scales overlap the codes
    (dict(scm=1, scn=1), EINVAL),            # cells (m, g + 1) and (m + 1, g) share a float
    (dict(sc=PD + (1 << 20) + 2), EALIGN),   # scales not 4-byte aligned
    (dict(scn=1 << 40), EUNSUPPORTED),
    (dict(sbn=1 << 30), EUNSUPPORTED),       # weight scale grid spanning 4 GiB
])
def test_gemm_quant_rejects(lib, kw, status):
    assert gq(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_block_gemm_quant")


def att(lib, q=PA, ldq=128, hq=64, hkv=8, t=300, d=128, kc=PB, ks=PC, vc=PB + (1 << 24), vs=PC + 4096, tb=128,
        fmt=E4M3, scale=0.088, out=PD, odt=BF16, ldo=128, ws=PD + (1 << 20), wsb=1 << 20):
    return lib.fp8_kv_decode_attention(q, ldq, hq, hkv, t, d, kc, ks, vc, vs, tb, fmt, scale, out, odt, ldo, ws,
                                       wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), EINVAL),
    (dict(ws=0), EINVAL),
    (dict(hq=60), EINVAL),                   # not a multiple of heads_kv
    (dict(hq=136), EUNSUPPORTED),            # 17 query heads per kv head
    (dict(t=0), EINVAL),
    (dict(d=64), EUNSUPPORTED),
    (dict(tb=64), EUNSUPPORTED),
    (dict(fmt=2), EINVAL),
    (dict(odt=5), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(q=PA + 8), EALIGN),
    (dict(ldq=132), EALIGN),
    (dict(out=PD + 2), EALIGN),
    (dict(wsb=16), EINVAL),                  # workspace too small
    (dict(out=PB + 64), EINVAL),             # out overlaps the K codes
    (dict(ws=PA), EINVAL),                   # workspace overlaps q
])
def test_attention_rejects(lib, kw, status):
    assert att(lib, **kw) == status


def att_noalloc(lib, q=PA, ldq=128, hq=64, hkv=8, t=300, d=128, kc=PB, ks=PC, vc=PB + (1 << 24), vs=PC + 4096,
                tb=128, fmt=E4M3, scale=0.088, out=PD, odt=BF16, ldo=128):
    return lib.fp8_kv_decode_attention_noalloc(q, ldq, hq, hkv, t, d, kc, ks, vc, vs, tb, fmt, scale, out, odt, ldo,
                                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), EINVAL),
    (dict(hq=60), EINVAL),
    (dict(d=64), EUNSUPPORTED),
    (dict(out=PB + 64), EINVAL),               # out overlaps the K codes
    (dict(hq=128, t=190 * 1408), EUNSUPPORTED),  # 24320 split partials: beyond the fixed 12 MiB
])
def test_attention_noalloc_rejects(lib, kw, status):
    assert att_noalloc(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_kv_decode_attention_noalloc")
    assert lib.fp8blk_last_error().decode().startswith("fp8_kv_decode_attention")


def test_attention_workspace_size(lib):
    lib.fp8_kv_decode_attention_workspace_size.restype = ctypes.c_size_t
    # 64 query heads, 131072 tokens: 94 splits of 1408 tokens (the last one
    # 128 tokens), 130 floats each
    assert lib.fp8_kv_decode_attention_workspace_size(64, 131072) == 64 * 94 * 130 * 4
    assert lib.fp8_kv_decode_attention_workspace_size(8, 1) == 8 * 1 * 130 * 4
    assert lib.fp8_kv_decode_attention_workspace_size(8, 1408) == 8 * 1 * 130 * 4
    assert lib.fp8_kv_decode_attention_workspace_size(8, 1409) == 8 * 2 * 130 * 4
    assert lib.fp8_kv_decode_attention_workspace_size(8, 2817) == 8 * 3 * 130 * 4
    assert lib.fp8_kv_decode_attention_workspace_size(0, 5) == 0


def qmx(lib, x=PA, dt=BF16, rows=4, cols=256, ldx=256, fmt=E4M3, qp=PB, ldq=256, s=PC, lds=8):
    return lib.fp8_quantize_mx(x, dt, rows, cols, ldx, fmt, qp, ldq, s, lds, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), EINVAL),
    (dict(fmt=2), EINVAL),
    (dict(dt=3), EINVAL),
    (dict(rows=-1), EINVAL),
    (dict(lds=7), EINVAL),                  # fewer than ceil(cols / 32) scale bytes per row
    (dict(ldq=128), EINVAL),
    (dict(x=PA + 2), EALIGN),
    (dict(ldq=264, cols=256), EALIGN),
    (dict(s=PB + 16), EINVAL),              # scales overlap the codes
])
def test_quantize_mx_rejects(lib, kw, status):
    assert qmx(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_quantize_mx")


def qst(lib, x=PA, dt=BF16, rows=4, cols=256, ldx=256, fmt=E4M3, s=PC, qp=PB, ldq=256, amax=PD):
    return lib.fp8_quantize_static(x, dt, rows, cols, ldx, fmt, s, qp, ldq, amax, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), EINVAL),
    (dict(s=0), EINVAL),                    # the scale is required
    (dict(fmt=2), EINVAL),
    (dict(dt=2), EINVAL),
    (dict(cols=-1), EINVAL),
    (dict(ldq=128), EINVAL),
    (dict(x=PA + 8), EALIGN),
    (dict(s=PC + 2), EALIGN),
    (dict(amax=PD + 1), EALIGN),
    (dict(amax=PC), EINVAL),                # amax_out is the scale
    (dict(s=PB + 64), EINVAL),              # the scale lies inside the codes
    (dict(rows=1 << 31), EUNSUPPORTED),
])
def test_quantize_static_rejects(lib, kw, status):
    assert qst(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_quantize_static")


def test_quantize_static_empty_without_amax_is_a_noop(lib):
    assert qst(lib, rows=0, amax=None) == OK
    assert qst(lib, cols=0, x=0, qp=0, amax=None) == OK     # no data pointers needed for an empty tensor


@pytest.mark.parametrize("args,status", [
    ((0, 4, E4M3, PB), EINVAL),
    ((PA, 0, E4M3, PB), EINVAL),            # empty history
    ((PA, 4, 7, PB), EINVAL),
    ((PA, 4, E4M3, 0), EINVAL),
    ((PA + 2, 4, E4M3, PB), EALIGN),
    ((PA, 4, E4M3, PA + 8), EINVAL),        # scale_out inside the history
])
def test_scale_from_history_rejects(lib, args, status):
    assert lib.fp8_scale_from_amax_history(*args, None) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_scale_from_amax_history")


def mxg(lib, M=256, N=256, K=256, a=PA, lda=256, sa=PB, ldsa=8, b=PC, ldb=256, sb=PB + 65536, ldsb=8,
        fa=E4M3, fb=E4M3, c=PD, cdt=BF16, ldc=256):
    return lib.fp8_mx_gemm(M, N, K, a, lda, sa, ldsa, b, ldb, sb, ldsb, fa, fb, c, cdt, ldc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(a=0), EINVAL),
    (dict(sb=0), EINVAL),
    (dict(fa=2), EINVAL),
    (dict(cdt=2), EINVAL),
    (dict(N=200), EUNSUPPORTED),
    (dict(ldsa=4), EINVAL),                 # fewer than K / 32 scale bytes per row
    (dict(ldsa=10), EALIGN),                # scale rows not 4-byte aligned
    (dict(sa=PB + 2), EALIGN),
    (dict(c=PA + 512), EINVAL),             # c overlaps a
])
def test_mx_gemm_rejects(lib, kw, status):
    assert mxg(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_mx_gemm")


def test_gemm_quant_empty_m_is_a_noop(lib):
    assert gq(lib, M=0) == OK


def test_gemm_empty_m_is_a_noop(lib):
    assert g(lib, M=0) == OK


def kvq(lib, kv=PA, h=2, t=300, d=128, sh=300 * 128, st=128, tb=128, fmt=E4M3, qp=PB, s=PC):
    return lib.fp8_kv_quantize(kv, h, t, d, sh, st, tb, fmt, qp, s, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kv=0), EINVAL),
    (dict(h=-1), EINVAL),
    (dict(d=0), EINVAL),
    (dict(tb=0), EINVAL),
    (dict(d=100, st=104, sh=300 * 104), EUNSUPPORTED),
    (dict(d=256, st=256, sh=300 * 256), EUNSUPPORTED),   # 128 x 256 > 16384 per group
    (dict(st=64), EINVAL),
    (dict(fmt=3), EINVAL),
    (dict(fmt=E5M2, st=64), EINVAL),      # E5M2 passes the format check
    (dict(kv=PA + 8), EALIGN),
    (dict(st=132), EALIGN),
    (dict(qp=PA + 4096), EINVAL),          # codes overlap the input
    (dict(s=PC + 2), EALIGN),              # scales not 4-byte aligned
])
def test_kv_quantize_rejects(lib, kw, status):
    assert kvq(lib, **kw) == status


def test_kv_empty_is_a_noop(lib):
    assert kvq(lib, t=0) == OK
    assert lib.fp8_kv_dequantize(PB, PC, 0, 300, 128, 128, E4M3, PD, None) == OK


@pytest.mark.parametrize("args,status", [
    ((0, PC, 2, 300, 128, 128, E4M3, PD), EINVAL),
    ((PB, PC, 2, 300, 128, 128, 2, PD), EINVAL),
    ((PB, PC, 2, 300, 128, 128, E5M2, PD + 2), EALIGN),
    ((PB, PC, 2, 300, 100, 128, E4M3, PD), EUNSUPPORTED),
    ((PB, PC, 2, 300, 128, 128, E4M3, PD + 2), EALIGN),
    ((PB, PC, 2, 300, 128, 128, E4M3, PB + 64), EINVAL),   # out overlaps the codes
    ((PB, PC + 2, 2, 300, 128, 128, E4M3, PD), EALIGN),    # scales not 4-byte aligned
])
def test_kv_dequantize_rejects(lib, args, status):
    assert lib.fp8_kv_dequantize(*args, None) == status


def test_gemm_rejects_huge_leading_dimension(lib):
    assert g(lib, lda=1 << 23) == EUNSUPPORTED


def qgd(lib, x=PA, xdt=BF16, M=64, N=512, K=512, ldx=512, ga=PER_TENSOR, fa=E4M3, b=PB, ldb=512, packed=0, sb=PC,
        gb=PER_TENSOR, sbn=0, sbk=0, fb=E4M3, c=PD, cdt=BF16, ldc=512, q=PD + (1 << 20), ldq=512, s=PD + (2 << 20),
        som=0, sok=0):
    return lib.fp8_quantize_gemm_decode(x, xdt, M, N, K, ldx, ga, fa, b, ldb, packed, sb, gb, sbn, sbk, fb, c, cdt,
                                        ldc, q, ldq, s, som, sok, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), EINVAL),
    (dict(c=0), EINVAL),
    (dict(xdt=2), EINVAL),
    (dict(cdt=2), EINVAL),
    (dict(gb=GROUP), EINVAL),
    (dict(ga=2), EINVAL),                       # activation scales are per tensor or 1x128
    (dict(packed=2), EINVAL),
    (dict(fa=2), EINVAL),
    (dict(M=0), EINVAL),
    (dict(M=65), EUNSUPPORTED),                 # prefill shapes take the two calls
    (dict(M=64, K=1152, ldx=1152, ldb=1152, ldq=1152), EUNSUPPORTED),   # per tensor: M * K above 65536
    (dict(N=192, ldc=192), EUNSUPPORTED),
    (dict(K=200, ldx=200, ldb=208, ldq=208), EUNSUPPORTED),
    (dict(ldx=256), EINVAL),
    (dict(ldq=256), EINVAL),
    (dict(x=PA + 8), EALIGN),
    (dict(ldx=516), EALIGN),
    (dict(s=PD + (2 << 20) + 2), EALIGN),
    (dict(q=PD + 1024), EINVAL),               # codes overlap the output
    (dict(c=PA + 1024), EINVAL),               # output overlaps the activations
    (dict(ga=GROUP, som=-1, sok=64), EINVAL),
    (dict(ga=GROUP, som=1, sok=1), EINVAL),    # two scales of the grid on one float
    (dict(ga=GROUP, som=1 << 40, sok=1), EUNSUPPORTED),
    (dict(ga=GROUP, som=4, sok=1, s=PD + 4), EINVAL),   # scale grid overlaps the output
    (dict(ga=GROUP, packed=1, ldb=7, c=PB + 1024), EINVAL),   # packed: ldb ignored, the N * K bytes still checked
])
def test_quantize_gemm_decode_rejects(lib, kw, status):
    assert qgd(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_quantize_gemm_decode")


def pk(lib, w=PA, N=256, K=256, ldw=256, out=PB):
    return lib.fp8_pack_weights_decode(w, N, K, ldw, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=0), EINVAL),
    (dict(out=0), EINVAL),
    (dict(N=0), EINVAL),
    (dict(K=-128), EINVAL),
    (dict(N=200), EUNSUPPORTED),
    (dict(K=200, ldw=208), EUNSUPPORTED),
    (dict(N=1 << 31), EUNSUPPORTED),
    (dict(ldw=128), EINVAL),
    (dict(w=PA + 8), EALIGN),
    (dict(ldw=264), EALIGN),
    (dict(out=PA + 4096), EINVAL),          # packed overlaps w
])
def test_pack_weights_decode_rejects(lib, kw, status):
    assert pk(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_pack_weights_decode")


def gp(lib, M=16, N=256, K=256, a=PA, lda=256, sa=PB, ga=GROUP, sam=1, sak=16, b=PC, sb=PB + 65536, gb=BLOCK,
       sbn=2, sbk=1, fa=E4M3, fb=E4M3, c=PD, cdt=BF16, ldc=256):
    return lib.fp8_block_gemm_packed(M, N, K, a, lda, sa, ga, sam, sak, b, sb, gb, sbn, sbk, fa, fb, c, cdt, ldc,
                                     None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=65), EUNSUPPORTED),             # prefill shapes take fp8_block_gemm
    (dict(b=0), EINVAL),
    (dict(c=0), EINVAL),
    (dict(cdt=3), EINVAL),
    (dict(N=200), EUNSUPPORTED),
    (dict(ldc=128), EINVAL),
    (dict(b=PC + 8), EALIGN),
    (dict(sb=PB + 65536 + 2), EALIGN),
    (dict(c=PC + 1024), EINVAL),            # c overlaps the packed weights (N * K bytes)
    (dict(fb=9), EINVAL),
    (dict(sak=1 << 30), EUNSUPPORTED),      # activation scale grid spanning 4 GiB
])
def test_gemm_packed_rejects(lib, kw, status):
    assert gp(lib, **kw) == status
    assert lib.fp8blk_last_error().decode().startswith("fp8_block_gemm_packed")


def test_gemm_packed_empty_m_is_a_noop(lib):
    assert gp(lib, M=0) == OK
