"""C-ABI checks of the latent-layer entry points that need no GPU: the
Python mirror of moe_latent_desc has the C layout, invalid descriptors and
calls are refused on the host before any launch, workspace sizes grow with
T and the AUTO path switches to MFMA above 3 tokens where it can."""
import ctypes
import os
import subprocess

import pytest

import quantized_expert_gemv_sigmoid_amd as moe
from test_abi import FAKE, L, ROOT  # noqa: F401  (L: the library fixture)

K3 = dict(n_experts=896, top_k=16, hidden=7168, latent=3584, d_ffn=3072, n_shared=2)
OPT = ("act", "path", "renorm", "routed_scale", "situ_b1", "situ_b2", "latent_norm", "rms_eps")
PTRS = ("router_w", "down", "w1_q", "w1_s", "w3_q", "w3_s", "w2_q", "w2_s", "norm_w", "up",
        "sh_w1", "sh_w3", "sh_w2")


def ldesc(**kw):
    t = {n: FAKE for n in PTRS}
    args = dict(K3)
    args.update({k: v for k, v in kw.items() if k in K3 or k in OPT})
    d = moe.make_latent_desc(args.pop("n_experts"), args.pop("top_k"), args.pop("hidden"),
                             args.pop("latent"), args.pop("d_ffn"), args.pop("n_shared"), t, **args)
    for k, v in kw.items():
        if k in t:
            setattr(d, k, v)
    return d


def call(L, d, T=1, x=FAKE, ws=(FAKE * 16, 1 << 40), out_mode=moe.OUT_F32, out_b=FAKE, out_f=FAKE):
    return L.moe_latent_layer(ctypes.byref(d) if d is not None else None, x, T, out_b, out_f,
                              out_mode, None, None, None, ws[0], ws[1], None)


def test_latent_desc_layout_matches_c(tmp_path):
    fields = [f for f, _ in moe.LatentDesc._fields_]
    prog = tmp_path / "layout.c"
    body = "\n".join(f'printf("%zu\\n", offsetof(moe_latent_desc, {f}));' for f in fields)
    prog.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "moe.h"\n'
                    'int main(void){ printf("%zu\\n", sizeof(moe_latent_desc));\n' + body + "\nreturn 0; }\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(prog), "-o", str(exe)])
    vals = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    assert vals[0] == ctypes.sizeof(moe.LatentDesc)
    for f, off in zip(fields, vals[1:]):
        assert getattr(moe.LatentDesc, f).offset == off, f


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=0), moe.EINVAL),
    (dict(hidden=7000), moe.EINVAL),
    (dict(latent=3583), moe.EINVAL),
    (dict(latent_norm=2), moe.EINVAL),
    (dict(rms_eps=-1e-5), moe.EINVAL),
    (dict(rms_eps=float("nan")), moe.EINVAL),
    (dict(act=5), moe.EINVAL),
    (dict(down=None), moe.EINVAL),
    (dict(up=None), moe.EINVAL),
    (dict(up=FAKE + 8), moe.EINVAL),
    (dict(down=FAKE + 2), moe.EINVAL),
    (dict(norm_w=FAKE + 2), moe.EINVAL),
    (dict(sh_w1=None), moe.EINVAL),
    (dict(hidden=8224), moe.EUNSUPPORTED),
    (dict(latent=4128), moe.EUNSUPPORTED),
    (dict(n_shared=4, d_ffn=4096), moe.EUNSUPPORTED),  # L + S F > 16384
    (dict(n_experts=2048), moe.EUNSUPPORTED),
])
def test_invalid_latent_descriptor_refused(L, kw, status):
    d = ldesc(**kw)
    assert call(L, d) == status
    assert L.moe_latent_workspace_bytes(ctypes.byref(d), 1) == 0


def test_latent_call_argument_checks(L):
    d = ldesc()
    need = L.moe_latent_workspace_bytes(ctypes.byref(d), 1)
    assert need > 0 and need % 256 == 0
    assert call(L, None) == moe.EINVAL
    assert call(L, d, x=None) == moe.EINVAL
    assert call(L, d, x=FAKE + 2) == moe.EINVAL
    assert call(L, d, T=-1) == moe.EINVAL
    assert call(L, d, ws=(FAKE * 16, need - 1)) == moe.EWORKSPACE
    assert call(L, d, ws=(FAKE * 16 + 64, need)) == moe.EINVAL
    assert call(L, d, out_mode=moe.OUT_BOTH, out_b=None) == moe.EINVAL
    assert call(L, d, T=0) == moe.OK
    # NULL norm weight means weight 1: a valid descriptor
    assert L.moe_latent_workspace_bytes(ctypes.byref(ldesc(norm_w=None)), 1) == need
    ev = (ctypes.c_void_p * moe.TIMED_EVENTS)(*([FAKE] * 5 + [None]))
    assert L.moe_latent_layer_timed(ctypes.byref(d), FAKE, 1, FAKE, FAKE, moe.OUT_BOTH, FAKE * 16,
                                    need, None, ev) == moe.EINVAL


def test_latent_workspace_monotone_and_paths(L):
    d = ldesc()
    ts = list(range(1, 80)) + [255, 256, 257, 1024, 4095, 4096, 4097]
    sizes = [L.moe_latent_workspace_bytes(ctypes.byref(d), t) for t in ts]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert moe.latent_path_for(d, 1) == moe.PATH_GEMV
    assert moe.latent_path_for(d, 3) == moe.PATH_GEMV
    assert moe.latent_path_for(d, 4) == moe.PATH_MFMA
    assert moe.latent_path_for(ldesc(path=moe.PATH_GEMV), 4096) == moe.PATH_GEMV
    # MFMA needs the hidden and latent widths to be multiples of 256
    assert moe.latent_path_for(ldesc(hidden=7200), 4096) == moe.PATH_GEMV
    d2 = ldesc(latent=3520, path=moe.PATH_MFMA)
    need = L.moe_latent_workspace_bytes(ctypes.byref(d2), 64)
    assert call(L, d2, T=64, ws=(FAKE * 16, need)) == moe.EUNSUPPORTED
