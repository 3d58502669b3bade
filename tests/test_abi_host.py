"""C-ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects bad arguments with the documented status
before making any HIP call. Only rejected calls are made here, so nothing is
ever launched. Pointers are fake, aligned or misaligned integers; the
library never dereferences a pointer on the host."""
import ctypes
import os
import re

import pytest

from combine_moe_finalize_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_finalize.h")

OK, NULLP, SHAPE, UNSUP, MISAL, FMT, ALIAS = 0, 1, 2, 3, 4, 5, 6

# fake device addresses, far apart and 256-byte aligned
G2, IDX, W, PK, SH, OUT, RES, GAM, RO, NRM, Q, S, ERR = [0x10_0000_0000 * (i + 1) for i in range(13)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe_finalize.so is not built (run python combine_moe_finalize_amd/build.py)")
    return B.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"moe_finalize", "moe_finalize_residual_rmsnorm",
                          "moe_finalize_quant_ue8m0", "moe_topk_packed_decode",
                          "moe_finalize_status_string", "moe_finalize_abi_version",
                          "moe_topk_sigmoid_gate", "moe_act_quant_fp8_ue8m0",
                          "moe_act_quant_fp8_amax", "moe_finalize_ep_combine",
                          "moe_allreduce_residual_rmsnorm", "moe_finalize_describe_launch"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.moe_finalize_abi_version() == 1
    for s in range(8):
        txt = lib.moe_finalize_status_string(s)
        assert txt and txt.decode()
    assert lib.moe_finalize_status_string(99).decode() == "unknown status"


def fin(lib, *, g2=G2, P=1024, idx=IDX, w=W, pk=None, sh=SH, rsf=2.5, out=OUT, T=4, H=4096,
        k=8, err=None):
    return lib.moe_finalize(g2, P, idx, w, pk, sh, rsf, out, T, H, k, err, None)


def test_finalize_shape_rules(lib):
    assert fin(lib, T=-1) == SHAPE
    assert fin(lib, P=-1) == SHAPE
    assert fin(lib, k=0) == SHAPE
    assert fin(lib, k=17) == SHAPE
    assert fin(lib, H=0) == SHAPE
    assert fin(lib, H=4100) == UNSUP             # not a multiple of 8
    assert fin(lib, H=(1 << 20) + 8) == UNSUP      # beyond the hidden limit
    assert fin(lib, P=1 << 31) == UNSUP          # rows are named by int32


def test_finalize_empty_batch_is_noop(lib):
    assert fin(lib, T=0, g2=None, idx=None, w=None, sh=None, out=None) == OK


def test_finalize_pointer_and_format_rules(lib):
    assert fin(lib, idx=None) == NULLP
    assert fin(lib, out=None) == NULLP
    assert fin(lib, g2=None) == NULLP
    assert fin(lib, g2=None, P=0) != NULLP       # P == 0 needs no buffer
    assert fin(lib, w=None, pk=None) == FMT      # neither format
    assert fin(lib, w=W, pk=PK) == FMT           # both formats


def test_finalize_alignment_rules(lib):
    assert fin(lib, g2=G2 + 8) == MISAL
    assert fin(lib, sh=SH + 2) == MISAL
    assert fin(lib, out=OUT + 4) == MISAL
    assert fin(lib, idx=IDX + 2) == MISAL
    assert fin(lib, w=W + 1) == MISAL
    assert fin(lib, err=ERR + 2) == MISAL


def test_finalize_alias_rules(lib):
    assert fin(lib, out=G2 + 4096 * 2 * 10) == ALIAS       # inside gemm2_out
    assert fin(lib, out=SH) == ALIAS
    assert fin(lib, out=IDX - 16) == ALIAS                  # straddles idx
    assert fin(lib, out=ERR, err=ERR) == ALIAS


def rms(lib, *, T=16, H=7168, k=8, res=RES, gam=GAM, ro=RO, nrm=NRM, sh=SH, w=W, pk=None,
        idx=IDX):
    return lib.moe_finalize_residual_rmsnorm(G2, 4096, idx, w, pk, sh, 2.5, res, gam, 1e-6,
                                             ro, nrm, T, H, k, None, None)


def test_rmsnorm_rules(lib):
    assert rms(lib, H=16392) == UNSUP               # beyond the on-chip row limit
    assert rms(lib, H=16384, res=None) == NULLP     # 16384 itself is allowed
    assert rms(lib, res=None) == NULLP
    assert rms(lib, gam=None) == NULLP
    assert rms(lib, nrm=None) == NULLP
    assert rms(lib, gam=GAM + 2) == MISAL
    assert rms(lib, ro=RES + 16) == ALIAS           # partial overlap with residual
    assert rms(lib, nrm=RO) == ALIAS                # normed == residual_out
    assert rms(lib, nrm=RES) == ALIAS
    assert rms(lib, ro=GAM) == ALIAS
    assert rms(lib, w=None, pk=None) == FMT
    assert rms(lib, T=0, res=None, gam=None, ro=None, nrm=None, sh=None, w=None,
               idx=None) == OK


def qnt(lib, *, T=8, H=7168, k=8, q=Q, s=S, w=W, pk=None):
    return lib.moe_finalize_quant_ue8m0(G2, 4096, IDX, w, pk, SH, 2.5, q, s, T, H, k, None, None)


def test_quant_rules(lib):
    assert qnt(lib, H=7168 + 8) == UNSUP            # not a multiple of 128
    assert qnt(lib, q=None) == NULLP
    assert qnt(lib, s=None) == NULLP
    assert qnt(lib, q=Q + 4) == MISAL
    assert qnt(lib, s=Q + 8 * 7168 - 1) == ALIAS    # scales overlap the codes
    assert qnt(lib, q=G2) == ALIAS
    assert qnt(lib, w=W, pk=PK) == FMT
    assert qnt(lib, T=0, q=None, s=None) == OK


def test_decode_rules(lib):
    d = lib.moe_topk_packed_decode
    assert d(PK, -1, IDX, W, None) == SHAPE
    assert d(PK, 0, None, None, None) == OK
    assert d(None, 8, IDX, W, None) == NULLP
    assert d(PK, 8, None, None, None) == NULLP
    assert d(PK + 2, 8, IDX, W, None) == MISAL
    assert d(PK, 8, PK + 16, W, None) == ALIAS
    assert d(PK, 8, IDX, IDX + 8, None) == ALIAS


def test_binding_rejects_flat_and_wrong_dtypes():
    import torch
    g2 = torch.zeros((256, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="2-D"):
        B.moe_finalize(g2, torch.zeros(16, dtype=torch.int32),
                       topk_weights=torch.zeros(16, dtype=torch.float32))
    idx = torch.zeros((8, 2), dtype=torch.int32)
    with pytest.raises(TypeError, match="int32"):           # fp32 passed as packed
        B.moe_finalize(g2, idx, topk_packed=torch.zeros((8, 2), dtype=torch.float32))
    with pytest.raises(TypeError, match="float32"):         # packed passed as fp32
        B.moe_finalize(g2, idx, topk_weights=torch.zeros((8, 2), dtype=torch.int32))
    with pytest.raises(ValueError, match="exactly one"):
        B.moe_finalize(g2, idx)
    with pytest.raises(ValueError, match="GPU"):             # CPU tensors never run
        B.moe_finalize(g2, idx, topk_weights=torch.zeros((8, 2), dtype=torch.float32))


def test_gate_rules(lib):
    g = lib.moe_topk_sigmoid_gate
    LG, ID, WT, PKD = G2, IDX, W, PK
    assert g(LG, -1, 256, 8, ID, WT, PKD, None) == SHAPE
    assert g(LG, 4, 0, 1, ID, WT, PKD, None) == SHAPE
    assert g(LG, 4, 256, 0, ID, WT, PKD, None) == SHAPE
    assert g(LG, 4, 256, 17, ID, WT, PKD, None) == SHAPE       # top_k above 16
    assert g(LG, 4, 4, 5, ID, WT, PKD, None) == SHAPE          # top_k above E
    assert g(LG, 4, 513, 8, ID, WT, PKD, None) == UNSUP        # E above the limit
    assert g(LG, 0, 256, 8, None, None, None, None) == OK
    assert g(None, 4, 256, 8, ID, WT, PKD, None) == NULLP
    assert g(LG, 4, 256, 8, None, WT, PKD, None) == NULLP      # ids are required
    assert g(LG + 2, 4, 256, 8, ID, WT, PKD, None) == MISAL
    assert g(LG, 4, 256, 8, LG + 64, WT, PKD, None) == ALIAS   # ids inside the logits
    assert g(LG, 4, 256, 8, ID, ID + 16, PKD, None) == ALIAS   # weights overlap ids


def test_act_quant_rules(lib):
    for fn in (lib.moe_act_quant_fp8_ue8m0, lib.moe_act_quant_fp8_amax):
        X, QQ, SS = G2, Q, S
        assert fn(X, -1, 7168, QQ, SS, None) == SHAPE
        assert fn(X, 4, 0, QQ, SS, None) == SHAPE
        assert fn(X, 4, 7168 + 8, QQ, SS, None) == UNSUP          # not a multiple of 128
        assert fn(X, 0, 7168, None, None, None) == OK
        assert fn(None, 4, 7168, QQ, SS, None) == NULLP
        assert fn(X, 4, 7168, None, SS, None) == NULLP
        assert fn(X, 4, 7168, QQ, None, None) == NULLP
        assert fn(X + 8, 4, 7168, QQ, SS, None) == MISAL
        assert fn(X, 4, 7168, QQ + 4, SS, None) == MISAL
        assert fn(X, 4, 7168, X + 64, SS, None) == ALIAS           # codes inside x
        assert fn(X, 4, 7168, QQ, QQ + 100, None) == ALIAS         # scales inside codes
    assert lib.moe_act_quant_fp8_amax(G2, 4, 7168, Q, S + 2, None) == MISAL


def test_ep_combine_rules(lib):
    c = lib.moe_finalize_ep_combine
    PP = G2
    assert c(PP, 0, SH, OUT, 4, 4096, None) == SHAPE
    assert c(PP, 65, SH, OUT, 4, 4096, None) == SHAPE
    assert c(PP, 4, SH, OUT, -1, 4096, None) == SHAPE
    assert c(PP, 4, SH, OUT, 4, 4100, None) == UNSUP
    assert c(PP, 4, SH, OUT, 0, 4096, None) == OK
    assert c(None, 4, SH, OUT, 4, 4096, None) == NULLP
    assert c(PP, 4, SH, None, 4, 4096, None) == NULLP
    assert c(PP + 8, 4, SH, OUT, 4, 4096, None) == MISAL
    assert c(PP, 4, SH, PP + 3 * 4 * 4096 * 2, 4, 4096, None) == ALIAS   # out = last partial
    assert c(PP, 4, SH, SH, 4, 4096, None) == ALIAS


def test_allreduce_rules(lib):
    c = lib.moe_allreduce_residual_rmsnorm
    T, H = 4, 4096
    tb = T * H * 2

    def ranks(*addrs):
        return (ctypes.c_void_p * len(addrs))(*addrs)

    rk = ranks(G2, G2 + 0x1_0000_0000, G2 + 0x2_0000_0000)
    assert c(rk, 0, RES, GAM, 1e-6, RO, NRM, T, H, None) == SHAPE
    assert c(rk, 17, RES, GAM, 1e-6, RO, NRM, T, H, None) == SHAPE
    assert c(rk, 3, RES, GAM, 1e-6, RO, NRM, -1, H, None) == SHAPE
    assert c(rk, 3, RES, GAM, 1e-6, RO, NRM, T, 0, None) == SHAPE
    assert c(rk, 3, RES, GAM, 1e-6, RO, NRM, T, 4100, None) == UNSUP
    assert c(rk, 3, RES, GAM, 1e-6, RO, NRM, T, 16392, None) == UNSUP
    assert c(rk, 3, RES, GAM, 1e-6, RO, NRM, 2 ** 31, 8, None) == UNSUP
    assert c(None, 3, RES, GAM, 1e-6, RO, NRM, 0, H, None) == OK          # empty batch
    assert c(None, 3, RES, GAM, 1e-6, RO, NRM, T, H, None) == NULLP
    assert c(ranks(G2, 0, G2 + 0x2_0000_0000), 3, RES, GAM, 1e-6, RO, NRM, T, H, None) == NULLP
    assert c(rk, 3, None, GAM, 1e-6, RO, NRM, T, H, None) == NULLP
    assert c(rk, 3, RES, GAM, 1e-6, RO, None, T, H, None) == NULLP
    assert c(ranks(G2, G2 + 8), 2, RES, GAM, 1e-6, RO, NRM, T, H, None) == MISAL
    assert c(rk, 3, RES, GAM + 4, 1e-6, RO, NRM, T, H, None) == MISAL
    assert c(rk, 3, RES, GAM, 1e-6, G2 + 0x1_0000_0000 + 64, NRM, T, H, None) == ALIAS
    assert c(rk, 3, RES, GAM, 1e-6, RES + 16, NRM, T, H, None) == ALIAS   # partial overlap
    assert c(rk, 3, RES, GAM, 1e-6, RO, RO + tb - 16, T, H, None) == ALIAS
    assert c(rk, 3, RES, GAM, 1e-6, RO, GAM, T, H, None) == ALIAS
    assert c(rk, 3, RES, GAM, 1e-6, RO, G2 + 0x2_0000_0000, T, H, None) == ALIAS


def test_err_flag_may_not_overlap_what_the_kernels_read(lib):
    """err_flag is written by the kernels: inside gemm2_out, the index map, the
    weights, the shared output, the residual or gamma it is an alias."""
    for err in (G2 + 64, IDX, W + 8, SH + 4):
        assert fin(lib, err=err) == ALIAS, hex(err)
    r = lib.moe_finalize_residual_rmsnorm
    for err in (RES + 4, GAM):
        assert r(G2, 1024, IDX, W, None, SH, 2.5, RES, GAM, 1e-6, RO, NRM, 4, 4096, 8, err,
                 None) == ALIAS
    q = lib.moe_finalize_quant_ue8m0
    assert q(G2, 1024, IDX, W, None, SH, 2.5, Q, S, 4, 4096, 8, IDX + 4, None) == ALIAS
