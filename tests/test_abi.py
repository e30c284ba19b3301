"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/moe.h declares, the Python mirror of moe_layer_desc has the C
layout, and invalid arguments are refused on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_expert_gemv_sigmoid_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from quantized_expert_gemv_sigmoid_amd import build
        build.build()
    return moe.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_desc_layout_matches_c(tmp_path):
    fields = [f for f, _ in moe.LayerDesc._fields_]
    prog = tmp_path / "layout.c"
    body = "\n".join(f'printf("%zu\\n", offsetof(moe_layer_desc, {f}));' for f in fields)
    prog.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\n'
                    'int main(void){ printf("%zu\\n", sizeof(moe_layer_desc));\n' + body + "\nreturn 0; }\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)])
    vals = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    assert vals[0] == ctypes.sizeof(moe.LayerDesc)
    for f, off in zip(fields, vals[1:]):
        assert getattr(moe.LayerDesc, f).offset == off, f


FAKE = 0x10000  # aligned, never dereferenced: every case below fails validation first


def desc(**kw):
    t = {n: FAKE for n in ("router_w", "w1_q", "w1_s", "w3_q", "w3_s", "w2_q", "w2_s",
                           "sh_w1", "sh_w3", "sh_w2")}
    args = dict(n_experts=896, top_k=16, d_model=3584, d_ffn=3072, n_shared=2)
    args.update({k: v for k, v in kw.items() if k in args or k in ("act", "path", "renorm", "routed_scale", "situ_b1", "situ_b2")})
    d = moe.make_desc(args.pop("n_experts"), args.pop("top_k"), args.pop("d_model"),
                      args.pop("d_ffn"), args.pop("n_shared"), t, **args)
    for k, v in kw.items():
        if k in t:
            setattr(d, k, v)
    return d


def call_layer(L, d, T=1, x=FAKE, ws=(FAKE * 16, 1 << 40), out_mode=moe.OUT_F32, out_b=FAKE,
               out_f=FAKE):
    return L.moe_layer(ctypes.byref(d) if d is not None else None, x, T, out_b, out_f, out_mode,
                       None, None, None, ws[0], ws[1], None)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), moe.EINVAL),
    (dict(top_k=900), moe.EINVAL),
    (dict(d_model=3583), moe.EINVAL),
    (dict(d_ffn=16), moe.EINVAL),
    (dict(n_shared=-1), moe.EINVAL),
    (dict(act=7), moe.EINVAL),
    (dict(path=9), moe.EINVAL),
    (dict(renorm=2), moe.EINVAL),
    (dict(situ_b1=0.0), moe.EINVAL),
    (dict(routed_scale=float("inf")), moe.EINVAL),
    (dict(w2_q=None), moe.EINVAL),
    (dict(w1_q=FAKE + 8), moe.EINVAL),
    (dict(router_w=FAKE + 4), moe.EINVAL),
    (dict(sh_w2=None), moe.EINVAL),
    (dict(n_experts=2048, top_k=16), moe.EUNSUPPORTED),
    (dict(top_k=80), moe.EUNSUPPORTED),
    (dict(d_model=8192), moe.EUNSUPPORTED),
    (dict(n_shared=9), moe.EUNSUPPORTED),
])
def test_invalid_descriptor_refused(L, kw, status):
    d = desc(**kw)
    assert call_layer(L, d) == status
    assert L.moe_workspace_bytes(ctypes.byref(d), 1) == 0


def test_null_descriptor(L):
    assert call_layer(L, None) == moe.EINVAL
    assert L.moe_workspace_bytes(None, 1) == 0


def test_call_argument_checks(L):
    d = desc()
    need = L.moe_workspace_bytes(ctypes.byref(d), 1)
    assert need > 0
    assert call_layer(L, d, x=None) == moe.EINVAL
    assert call_layer(L, d, x=FAKE + 2) == moe.EINVAL
    assert call_layer(L, d, T=-1) == moe.EINVAL
    assert call_layer(L, d, T=(1 << 20) + 1) == moe.EUNSUPPORTED
    assert call_layer(L, d, ws=(FAKE * 16, need - 1)) == moe.EWORKSPACE
    assert call_layer(L, d, ws=(FAKE * 16 + 128, need)) == moe.EINVAL
    assert call_layer(L, d, ws=(None, need)) == moe.EINVAL
    assert call_layer(L, d, out_mode=5) == moe.EINVAL
    assert call_layer(L, d, out_mode=moe.OUT_BF16, out_b=None) == moe.EINVAL
    assert call_layer(L, d, out_mode=moe.OUT_BOTH, out_f=None) == moe.EINVAL
    assert call_layer(L, d, out_mode=moe.OUT_F32, out_f=FAKE + 4) == moe.EINVAL
    # T = 0 is a no-op that touches nothing
    assert call_layer(L, d, T=0) == moe.OK
    assert L.moe_route(ctypes.byref(d), FAKE, 1, None, FAKE, None, FAKE * 16, need, None) == moe.EINVAL
    assert L.moe_expert_forward(ctypes.byref(d), FAKE, 1, FAKE, FAKE, 3, None, FAKE, moe.OUT_F32,
                                FAKE * 16, need, None) == moe.EINVAL


def test_workspace_monotone_and_paths(L):
    d = desc()
    # every T: one call sized for max_tokens serves any smaller T
    ts = list(range(1, 300)) + [511, 512, 513, 1023, 1024, 1025, 2048, 4095, 4096, 4097, 8192]
    sizes = [L.moe_workspace_bytes(ctypes.byref(d), t) for t in ts]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert sizes[0] % 256 == 0
    assert moe.path_for(d, 1) == moe.PATH_GEMV
    # AUTO at the Kimi-K3 shape: GEMV up to 12 tokens, the grouped GEMM from 13
    assert moe.path_for(d, 12) == moe.PATH_GEMV
    assert moe.path_for(d, 13) == moe.PATH_MFMA
    assert moe.path_for(desc(path=moe.PATH_GEMV), 4096) == moe.PATH_GEMV
    assert moe.path_for(desc(path=moe.PATH_MFMA), 1) == moe.PATH_MFMA


def test_status_strings(L):
    for s in (moe.OK, moe.EINVAL, moe.EUNSUPPORTED, moe.EWORKSPACE, moe.EHIP):
        assert moe.status_str(s) not in ("", "unknown status")
    assert moe.status_str(12345) == "unknown status"


def test_router_wait_setting(L):
    assert L.moe_set_one_token_router_wait(-1) == moe.EINVAL
    assert L.moe_set_one_token_router_wait(0) == moe.OK
    assert L.moe_set_one_token_router_wait(50) == moe.OK


def test_mfma_route_outside_its_range_refused(L):
    """moe_route with an explicit MFMA path checks the path's range before any
    launch, as the expert entry points do: d = 3200 is not a multiple of 256."""
    d = desc(d_model=3200, path=moe.PATH_MFMA)
    need = L.moe_workspace_bytes(ctypes.byref(d), 4)
    assert need > 0
    assert L.moe_route(ctypes.byref(d), FAKE, 4, FAKE, FAKE, None, FAKE * 16, need, None) == moe.EUNSUPPORTED
    assert call_layer(L, d, T=4, ws=(FAKE * 16, need)) == moe.EUNSUPPORTED
    assert L.moe_expert_forward(ctypes.byref(d), FAKE, 4, FAKE, FAKE, 1, None, FAKE, moe.OUT_F32,
                                FAKE * 16, need, None) == moe.EUNSUPPORTED
    # AUTO stays on the GEMV path there
    assert moe.path_for(desc(d_model=3200), 4096) == moe.PATH_GEMV


def test_fp16_h_paths_need_situ_within_fp16(L):
    """SiTU bounds |h| by b1*b2: above 65504 (the largest fp16) the fp16-H MFMA
    path is refused when asked for and AUTO keeps the fp32-H GEMV kernels."""
    big = desc(situ_b1=4.0, situ_b2=20000.0, path=moe.PATH_MFMA)
    need = L.moe_workspace_bytes(ctypes.byref(big), 4096)
    assert need > 0
    assert call_layer(L, big, T=4096, ws=(FAKE * 16, need)) == moe.EUNSUPPORTED
    assert moe.path_for(desc(situ_b1=4.0, situ_b2=20000.0), 4096) == moe.PATH_GEMV
    assert moe.path_for(desc(situ_b1=4.0, situ_b2=16376.0), 4096) == moe.PATH_MFMA  # 65504 exactly
    assert moe.path_for(desc(act=moe.ACT_SWIGLU), 4096) == moe.PATH_MFMA
