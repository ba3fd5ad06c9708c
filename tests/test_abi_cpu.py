"""The C-ABI library loads, exports what include/infv2.h declares, and rejects
bad arguments before touching the GPU (CPU only: no compute call here ever
passes validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest
import torch

import trainable_block_sparse_mean_amd as tb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infv2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tb.LIB_PATH), reason="libinfv2.so not built")

FAKE = 0x10000      # aligned, non-null; only ever passed where validation fails first
FAKE_MIS = 0x10004  # misaligned

# calls with fake pointers must never reach a kernel; as a second guard they
# only run where no GPU is visible
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer validation tests run GPU-less only")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(infv2_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ["infv2_compress_k", "infv2_select_blocks", "infv2_sparse_attn_fwd", "infv2_dense_attn_fwd",
              "infv2_attn_fwd", "infv2_sparse_attn_bwd", "infv2_status_string", "infv2_decode_compress_append",
              "infv2_decode_select", "infv2_decode_attn", "infv2_compress_v", "infv2_compressed_attn_fwd",
              "infv2_decode_compressed_attn", "infv2_mixed_attn_fwd", "infv2_attn_path",
              "infv2_attn_fwd_noalloc", "infv2_decode_select_attn"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tb.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(tb.SIGNATURES) == set(declared_functions())


def test_status_strings_and_version():
    lib = tb.load_library()
    assert lib.infv2_abi_version() == 1
    assert lib.infv2_status_string(0) == b"ok"
    assert lib.infv2_status_string(3) == b"workspace missing or too small"
    assert lib.infv2_status_string(99) == b"unknown status"


def _sparse(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, idx=FAKE, out=FAKE, lse=None, B=1, H_q=32, H_kv=2, S_q=128, S_k=128,
             D=128, bs=64, topk=4, n_init=1, n_local=2, scale=0.0, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return lib.infv2_sparse_attn_fwd(a["q"], a["k"], a["v"], a["idx"], a["out"], a["lse"], a["B"], a["H_q"],
                                     a["H_kv"], a["S_q"], a["S_k"], a["D"], a["bs"], a["topk"], a["n_init"],
                                     a["n_local"], a["scale"], a["ws"], a["wsb"], a["stream"])


@no_gpu
def test_sparse_validation_codes():
    lib = tb.load_library()
    assert _sparse(lib, H_q=31) == tb.ERR_INVALID              # H_q % H_kv
    assert _sparse(lib, S_q=129) == tb.ERR_INVALID             # S_q > S_k
    assert _sparse(lib, n_local=0) == tb.ERR_INVALID           # the diagonal block must be attended
    assert _sparse(lib, n_init=-1) == tb.ERR_INVALID
    assert _sparse(lib, topk=-1) == tb.ERR_INVALID
    assert _sparse(lib, B=-1) == tb.ERR_INVALID
    assert _sparse(lib, D=64) == tb.ERR_UNSUPPORTED
    assert _sparse(lib, bs=32) == tb.ERR_UNSUPPORTED
    assert _sparse(lib, topk=257) == tb.ERR_UNSUPPORTED
    assert _sparse(lib, H_q=64, H_kv=2) == tb.ERR_UNSUPPORTED  # G = 32 > 16
    assert _sparse(lib, q=None) == tb.ERR_INVALID
    assert _sparse(lib, out=FAKE_MIS) == tb.ERR_INVALID
    # empty inputs are valid no-ops (return before any HIP call)
    assert _sparse(lib, B=0) == tb.OK
    assert _sparse(lib, S_q=0) == tb.OK


def test_workspace_sizes():
    lib = tb.load_library()
    # long queries need no workspace; short ones (decode) hold split-KV
    # partials: nsplit x B x H_q x S_q rows of 132 floats
    assert lib.infv2_sparse_workspace_bytes(1, 32, 2, 32768, 32768, 128, 64, 64) == 0
    assert lib.infv2_dense_workspace_bytes(2, 8, 1, 64, 64, 128) == 0
    dec = lib.infv2_sparse_workspace_bytes(16, 32, 2, 1, 32768, 128, 64, 64)
    assert dec == 8 * 16 * 32 * 1 * 132 * 4                    # 8 splits: 256 workgroups over 32 windows
    one = lib.infv2_sparse_workspace_bytes(1, 32, 2, 1, 32768, 128, 64, 64)
    assert one == 16 * 1 * 32 * 1 * 132 * 4                    # at most 16 splits
    assert lib.infv2_sparse_workspace_bytes(1, 32, 2, 1, 1000, 128, 64, 4) == 0   # one split: no partials
    dense = lib.infv2_attn_workspace_bytes(1, 32, 2, 4096, 4096, 128, 64, 16, 4096)
    sparse = lib.infv2_attn_workspace_bytes(1, 32, 2, 4097, 4097, 128, 64, 16, 4096)
    assert dense == lib.infv2_dense_workspace_bytes(1, 32, 2, 4096, 4096, 128)
    kc = 2 * 65 * 128 * 2                       # bf16 [1][2][ceil(4097/64)][128]
    idx = 2 * 4097 * 16 * 4                     # int32 [1][2][4097][16]
    rnd = lambda x: (x + 255) // 256 * 256
    assert sparse == rnd(kc) + rnd(idx) + lib.infv2_sparse_workspace_bytes(1, 32, 2, 4097, 4097, 128, 64, 16)


@no_gpu
def test_other_entry_points_validate():
    lib = tb.load_library()
    assert lib.infv2_compress_k(FAKE, FAKE, 1, 2, 100, 96, 64, None) == tb.ERR_UNSUPPORTED
    assert lib.infv2_compress_k(FAKE, None, 1, 2, 100, 128, 64, None) == tb.ERR_INVALID
    assert lib.infv2_compress_k(FAKE, FAKE, 1, 0, 100, 128, 64, None) == tb.ERR_INVALID
    assert lib.infv2_compress_k(FAKE, FAKE, 0, 2, 100, 128, 64, None) == tb.OK
    sel = lib.infv2_select_blocks
    assert sel(FAKE, FAKE, FAKE, None, 1, 32, 2, 10, 4065 * 64, 128, 64, 8, 1, 2, 0.0, None) == tb.ERR_UNSUPPORTED
    assert sel(FAKE, FAKE, FAKE, FAKE_MIS, 1, 32, 2, 10, 2000, 128, 64, 8, 1, 2, 0.0, None) == tb.ERR_INVALID
    assert sel(FAKE, FAKE, None, None, 1, 32, 2, 10, 2000, 128, 64, 8, 1, 2, 0.0, None) == tb.ERR_INVALID
    assert sel(FAKE, FAKE, FAKE, None, 1, 32, 2, 10, 2000, 128, 64, 8, 1, 0, 0.0, None) == tb.ERR_INVALID
    dense = lib.infv2_dense_attn_fwd
    assert dense(FAKE, FAKE, FAKE, FAKE, None, 1, 8, 1, 64, 64, 128, 0.0, 2, FAKE, 1 << 20, None) == tb.ERR_INVALID
    assert dense(FAKE, FAKE, None, FAKE, None, 1, 8, 1, 64, 64, 128, 0.0, 1, FAKE, 16, None) == tb.ERR_INVALID
    assert dense(FAKE, FAKE, FAKE, FAKE, FAKE_MIS, 1, 8, 1, 64, 64, 128, 0.0, 1, FAKE, 16, None) == tb.ERR_INVALID
    assert dense(FAKE, FAKE, FAKE, FAKE, None, 1, 8, 3, 64, 64, 128, 0.0, 1, FAKE, 1 << 20, None) == tb.ERR_INVALID
    sw = lib.infv2_attn_fwd
    # dense branch (S_k <= switch_len) and sparse branch both validate first
    assert sw(FAKE, FAKE, FAKE, None, None, None, 1, 32, 2, 64, 64, 128, 64, 4, 1, 2, 0.0, 64, FAKE, 8,
              None) == tb.ERR_INVALID
    assert sw(FAKE, FAKE, FAKE, FAKE, None, None, 1, 32, 2, 128, 128, 128, 64, 4, 1, 2, 0.0, 64, FAKE, 8,
              None) == tb.ERR_WORKSPACE
    assert sw(FAKE, FAKE, FAKE, FAKE, None, None, 1, 32, 2, 128, 128, 128, 64, 4, 1, 0, 0.0, 64, FAKE, 1 << 30,
              None) == tb.ERR_INVALID


def test_binding_refuses_cpu_tensors():
    q = torch.zeros(1, 2, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        tb.compress_k(q)
    with pytest.raises(ValueError, match="GPU"):
        tb.dense_attn_fwd(q, q[:, :1].contiguous(), q[:, :1].contiguous())


def test_binding_raises_when_library_missing(tmp_path, monkeypatch):
    monkeypatch.setattr(tb, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        tb.load_library(str(tmp_path / "nope.so"))


def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, idx=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1,
             H_q=32, H_kv=2, S_q=128, S_k=128, D=128, bs=64, topk=4, n_init=1, n_local=2, scale=0.0, ws=FAKE,
             wsb=0, stream=None)
    a.update(kw)
    return lib.infv2_sparse_attn_bwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"], a["idx"], a["dq"],
                                     a["dk"], a["dv"], a["B"], a["H_q"], a["H_kv"], a["S_q"], a["S_k"], a["D"],
                                     a["bs"], a["topk"], a["n_init"], a["n_local"], a["scale"], a["ws"], a["wsb"],
                                     a["stream"])


@no_gpu
def test_backward_validation_codes():
    lib = tb.load_library()
    assert _bwd(lib, H_q=31) == tb.ERR_INVALID                 # H_q % H_kv
    assert _bwd(lib, S_q=129) == tb.ERR_INVALID                # S_q > S_k
    assert _bwd(lib, n_local=0) == tb.ERR_INVALID
    assert _bwd(lib, lse=None) == tb.ERR_INVALID               # the forward's lse is required
    assert _bwd(lib, dout=FAKE_MIS) == tb.ERR_INVALID
    assert _bwd(lib, dk=None) == tb.ERR_INVALID
    assert _bwd(lib, D=64) == tb.ERR_UNSUPPORTED
    assert _bwd(lib, H_q=64, H_kv=2) == tb.ERR_UNSUPPORTED      # G = 32 > 16
    assert _bwd(lib, S_q=10, S_k=4064 * 64 + 1) == tb.ERR_UNSUPPORTED   # more key blocks than LDS holds
    assert _bwd(lib, ws=None) == tb.ERR_WORKSPACE
    assert _bwd(lib, wsb=1024) == tb.ERR_WORKSPACE
    assert _bwd(lib, B=0) == tb.OK                             # nothing to write


def test_backward_workspace_sizes():
    lib = tb.load_library()
    # D (4 bytes per row and head, rounded to 256) + one bit per (KV head, block, token)
    # (rounded to 256) + fp32 dk/dv partials of 16 token pieces per block from 3 * 4096 queries on
    assert lib.infv2_sparse_bwd_workspace_bytes(1, 32, 2, 32768, 32768, 128, 64, 64) == \
        32 * 32768 * 4 + 2 * 512 * 1024 * 4 + 2 * 512 * 16 * (2 * 64 * 128 * 4)
    assert lib.infv2_sparse_bwd_workspace_bytes(2, 6, 3, 37, 1000, 128, 64, 5) == \
        ((2 * 6 * 37 * 4 + 255) // 256) * 256 + 2 * 3 * 16 * 2 * 4
    assert lib.infv2_sparse_bwd_workspace_bytes(1, 32, 2, 10, 10, 64, 64, 4) == 0   # unsupported D


@no_gpu
def test_sparse_block_limit_is_what_lds_holds():
    lib = tb.load_library()
    # 4064 blocks fill the 160 KB of LDS (ring, control words, union list); 4065 is the first refused
    assert _sparse(lib, S_q=10, S_k=4064 * 64 + 1) == tb.ERR_UNSUPPORTED
    assert _dec_attn(lib, max_blocks=4065) == tb.ERR_UNSUPPORTED



def _dec_attn(lib, **kw):
    a = dict(q=FAKE, kp=FAKE, vp=FAKE, table=FAKE, lens=FAKE, idx=FAKE, out=FAKE, lse=FAKE, B=16, H_q=32, H_kv=2,
             D=128, bs=64, max_blocks=512, num_pages=8192, topk=64, n_init=1, n_local=2, scale=0.0, ws=FAKE,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.infv2_decode_attn(a["q"], a["kp"], a["vp"], a["table"], a["lens"], a["idx"], a["out"], a["lse"],
                                 a["B"], a["H_q"], a["H_kv"], a["D"], a["bs"], a["max_blocks"], a["num_pages"],
                                 a["topk"], a["n_init"], a["n_local"], a["scale"], a["ws"], a["wsb"], a["stream"])


def _dec_fused(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, kp=FAKE, vp=FAKE, table=FAKE, lens=FAKE, idx=FAKE, score=None, out=FAKE, lse=FAKE,
             B=16, H_q=32, H_kv=2, D=128, bs=64, max_blocks=512, num_pages=8192, topk=64, n_init=1, n_local=2,
             scale=0.0, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.infv2_decode_select_attn(a["q"], a["kc"], a["kp"], a["vp"], a["table"], a["lens"], a["idx"],
                                        a["score"], a["out"], a["lse"], a["B"], a["H_q"], a["H_kv"], a["D"], a["bs"],
                                        a["max_blocks"], a["num_pages"], a["topk"], a["n_init"], a["n_local"],
                                        a["scale"], a["ws"], a["wsb"], a["stream"])


@no_gpu
def test_decode_select_attn_validation_codes():
    """The fused decode call refuses what the selection or the attention
    call would refuse, before any launch."""
    lib = tb.load_library()
    assert _dec_fused(lib, H_q=31) == tb.ERR_INVALID               # H_q % H_kv
    assert _dec_fused(lib, kc=None) == tb.ERR_INVALID
    assert _dec_fused(lib, table=None) == tb.ERR_INVALID
    assert _dec_fused(lib, lens=FAKE + 2) == tb.ERR_INVALID        # int32 arrays must be 4-byte aligned
    assert _dec_fused(lib, idx=None) == tb.ERR_INVALID             # topk > 0 needs the selection's output
    assert _dec_fused(lib, score=FAKE + 4) == tb.ERR_INVALID       # scores must be 16-byte aligned
    assert _dec_fused(lib, num_pages=0) == tb.ERR_INVALID
    assert _dec_fused(lib, n_local=0) == tb.ERR_INVALID
    assert _dec_fused(lib, D=64) == tb.ERR_UNSUPPORTED
    assert _dec_fused(lib, max_blocks=2049) == tb.ERR_UNSUPPORTED  # the decode selection's limit
    assert _dec_fused(lib, topk=257) == tb.ERR_UNSUPPORTED
    assert _dec_fused(lib, ws=None) == tb.ERR_WORKSPACE
    assert _dec_fused(lib, wsb=1024) == tb.ERR_WORKSPACE
    assert _dec_fused(lib, B=0) == tb.OK


@no_gpu
def test_decode_validation_codes():
    lib = tb.load_library()
    assert _dec_attn(lib, H_q=31) == tb.ERR_INVALID                # H_q % H_kv
    assert _dec_attn(lib, max_blocks=0) == tb.ERR_INVALID
    assert _dec_attn(lib, num_pages=0) == tb.ERR_INVALID
    assert _dec_attn(lib, table=None) == tb.ERR_INVALID
    assert _dec_attn(lib, lens=FAKE + 2) == tb.ERR_INVALID         # int32 arrays must be 4-byte aligned
    assert _dec_attn(lib, kp=FAKE_MIS) == tb.ERR_INVALID
    assert _dec_attn(lib, n_local=0) == tb.ERR_INVALID
    assert _dec_attn(lib, D=64) == tb.ERR_UNSUPPORTED
    assert _dec_attn(lib, bs=32) == tb.ERR_UNSUPPORTED
    assert _dec_attn(lib, max_blocks=4097) == tb.ERR_UNSUPPORTED   # more blocks than the sparse kernel's LDS holds
    assert _dec_attn(lib, ws=None) == tb.ERR_WORKSPACE
    assert _dec_attn(lib, wsb=1024) == tb.ERR_WORKSPACE
    assert _dec_attn(lib, B=0) == tb.OK
    sel = lambda **kw: lib.infv2_decode_select(kw.get("q", FAKE), FAKE, kw.get("lens", FAKE), FAKE, None,
                                               kw.get("B", 16), 32, 2, 128, 64, kw.get("max_blocks", 512),
                                               kw.get("topk", 64), 1, 2, 0.0, None)
    assert sel(lens=None) == tb.ERR_INVALID
    assert sel(max_blocks=2049) == tb.ERR_UNSUPPORTED              # scores of more blocks than LDS holds
    assert sel(topk=257) == tb.ERR_UNSUPPORTED
    assert sel(B=0) == tb.OK
    app = lambda **kw: lib.infv2_decode_compress_append(FAKE, kw.get("table", FAKE), FAKE, FAKE, FAKE, 16, 2, 128,
                                                        64, 512, kw.get("num_pages", 100), kw.get("max_new", 1),
                                                        None)
    assert app(table=None) == tb.ERR_INVALID
    assert app(num_pages=0) == tb.ERR_INVALID
    assert app(max_new=513) == tb.ERR_INVALID                      # more new blocks than a sequence holds
    assert app(max_new=0) == tb.OK


def test_decode_workspace_sizes():
    lib = tb.load_library()
    # B * H_kv = 32 windows of one query: 8 splits of the block list (about
    # one workgroup per CU), each writing 132 fp32 per (batch, query head)
    assert lib.infv2_decode_attn_workspace_bytes(16, 32, 2, 128, 64, 512, 64) == 8 * 16 * 32 * 132 * 4
    assert lib.infv2_decode_attn_workspace_bytes(16, 32, 2, 64, 64, 512, 64) == 0      # unsupported D


def _cmp_attn(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o_sparse=None, out=FAKE, lse=None, B=1, H_q=32, H_kv=2, S_q=4096,
             S_k=4096, D=128, bs=64, scale=0.0, ws=0.5, wc=0.5)
    a.update(kw)
    return lib.infv2_compressed_attn_fwd(a["q"], a["kc"], a["vc"], a["o_sparse"], a["out"], a["lse"], a["B"],
                                         a["H_q"], a["H_kv"], a["S_q"], a["S_k"], a["D"], a["bs"], a["scale"],
                                         a["ws"], a["wc"], None)


@no_gpu
def test_compressed_branch_validation_codes():
    lib = tb.load_library()
    assert lib.infv2_compress_v(FAKE, FAKE, 1, 2, 100, 96, 64, None) == tb.ERR_UNSUPPORTED
    assert lib.infv2_compress_v(FAKE, None, 1, 2, 100, 128, 64, None) == tb.ERR_INVALID
    assert lib.infv2_compress_v(FAKE, FAKE, 0, 2, 100, 128, 64, None) == tb.OK
    assert _cmp_attn(lib, H_q=31) == tb.ERR_INVALID
    assert _cmp_attn(lib, S_q=4097) == tb.ERR_INVALID               # more queries than keys
    assert _cmp_attn(lib, vc=None) == tb.ERR_INVALID
    assert _cmp_attn(lib, out=FAKE_MIS) == tb.ERR_INVALID
    assert _cmp_attn(lib, o_sparse=FAKE_MIS) == tb.ERR_INVALID
    assert _cmp_attn(lib, lse=FAKE + 4) == tb.ERR_INVALID
    assert _cmp_attn(lib, ws=float("nan")) == tb.ERR_INVALID
    assert _cmp_attn(lib, wc=float("inf")) == tb.ERR_INVALID
    assert _cmp_attn(lib, bs=0) == tb.ERR_INVALID
    assert _cmp_attn(lib, bs=32) == tb.ERR_UNSUPPORTED
    assert _cmp_attn(lib, D=64) == tb.ERR_UNSUPPORTED
    assert _cmp_attn(lib, H_q=34, H_kv=2) == tb.ERR_UNSUPPORTED       # 17 heads per group
    assert _cmp_attn(lib, S_q=0) == tb.OK
    dec = lambda **kw: lib.infv2_decode_compressed_attn(FAKE, FAKE, FAKE, kw.get("lens", FAKE), None, FAKE, None,
                                                        kw.get("B", 16), 32, 2, 128, kw.get("bs", 64),
                                                        kw.get("max_blocks", 512), 0.0, kw.get("ws", 0.0), 1.0,
                                                        None)
    assert dec(lens=None) == tb.ERR_INVALID
    assert dec(lens=FAKE + 2) == tb.ERR_INVALID
    assert dec(max_blocks=0) == tb.ERR_INVALID
    assert dec(ws=float("nan")) == tb.ERR_INVALID
    assert dec(bs=128) == tb.ERR_UNSUPPORTED
    assert dec(B=0) == tb.OK


@no_gpu
def test_c_program_compiles_links_and_validates(tmp_path):
    """The header is plain C99 (warnings are errors) and a C program links
    against the library and gets validation codes back (no GPU call)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "c_abi_smoke"
    libdir = os.path.dirname(tb.LIB_PATH)
    src = os.path.join(ROOT, "tests", "c_abi_smoke.c")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), src,
           "-o", str(exe), "-L", libdir, "-linfv2", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "c abi ok" in run.stdout, (run.returncode, run.stdout, run.stderr)


@no_gpu
def test_mixed_attn_validation_codes():
    lib = tb.load_library()
    mix = lambda **kw: lib.infv2_mixed_attn_fwd(
        kw.get("q", FAKE), FAKE, FAKE, kw.get("idx", FAKE), kw.get("kc", FAKE), FAKE, FAKE, kw.get("lse", None),
        kw.get("B", 1), 32, 2, kw.get("S_q", 4096), 4096, kw.get("D", 128), 64, kw.get("topk", 8), 1,
        kw.get("n_local", 2), 0.0, kw.get("ws", 0.5), 0.5, kw.get("wsp", None), kw.get("wsb", 0), None)
    assert mix(kc=None) == tb.ERR_INVALID
    assert mix(idx=None) == tb.ERR_INVALID                       # topk > 0 needs the selection
    assert mix(lse=FAKE + 8) == tb.ERR_INVALID
    assert mix(ws=float("nan")) == tb.ERR_INVALID
    assert mix(n_local=0) == tb.ERR_INVALID
    assert mix(D=64) == tb.ERR_UNSUPPORTED
    assert mix(topk=300) == tb.ERR_UNSUPPORTED
    assert mix(S_q=1) == tb.ERR_WORKSPACE                        # one query row: split partials needed
    assert mix(B=0) == tb.OK


@no_gpu
def test_noalloc_switch_refuses_shapes_beyond_its_scratch():
    lib = tb.load_library()

    def call(**kw):
        a = dict(B=1, H_q=32, H_kv=2, S_q=131072, S_k=131072, topk=128, switch_len=0)
        a.update(kw)
        return lib.infv2_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, None, None, a["B"], a["H_q"], a["H_kv"], a["S_q"],
                                          a["S_k"], 128, 64, a["topk"], 1, 2, 0.0, a["switch_len"], None)
    # 128k tokens with top-128: 134 MB of block indices, beyond the 32 MiB scratch
    need = lib.infv2_attn_workspace_bytes(1, 32, 2, 131072, 131072, 128, 64, 128, 0)
    assert need > 32 << 20
    assert call() == tb.ERR_WORKSPACE
    assert call(H_q=31) == tb.ERR_INVALID
    assert call(B=0) == tb.OK
    assert call(S_k=4064 * 64 + 1, S_q=10) == tb.ERR_UNSUPPORTED   # beyond the 4064 blocks selection keeps


@no_gpu
def test_launch_grid_limits_are_refused_before_any_launch():
    lib = tb.load_library()
    # (batch, kv head) pairs go in gridDim.y: 65535 at most
    assert _bwd(lib, B=65536, H_q=1, H_kv=1, S_q=1, S_k=1) == tb.ERR_UNSUPPORTED
    assert _bwd(lib, B=32768, H_q=2, H_kv=2, S_q=1, S_k=1) == tb.ERR_UNSUPPORTED
    assert _sparse(lib, B=65536, H_q=1, H_kv=1, S_q=1, S_k=1) == tb.ERR_UNSUPPORTED
    assert lib.infv2_compress_k(FAKE, FAKE, 65536, 1, 64, 128, 64, None) == tb.ERR_UNSUPPORTED
    assert _dec_attn(lib, B=65536, H_q=1, H_kv=1, max_blocks=1) == tb.ERR_UNSUPPORTED
    # work-items: B * H_kv * S_k <= 2^25
    assert _bwd(lib, B=512, H_q=2, H_kv=2, S_q=1, S_k=32769) == tb.ERR_UNSUPPORTED
    assert _sparse(lib, B=1024, H_q=1, H_kv=1, S_q=1, S_k=32769) == tb.ERR_UNSUPPORTED
    assert lib.infv2_compress_k(FAKE, FAKE, 512, 2, 32769, 128, 64, None) == tb.ERR_UNSUPPORTED
    # at the limit the shape is accepted (and then stopped by the missing workspace)
    assert _bwd(lib, B=512, H_q=2, H_kv=2, S_q=1, S_k=32768, ws=None) == tb.ERR_WORKSPACE
    assert _bwd(lib, B=65535, H_q=1, H_kv=1, S_q=1, S_k=1, ws=None) == tb.ERR_WORKSPACE


def test_switch_path_rule_lives_in_the_library():
    lib = tb.load_library()
    assert lib.infv2_attn_path(4096, 4096) == tb.PATH_DENSE
    assert lib.infv2_attn_path(4097, 4096) == tb.PATH_SPARSE
    assert lib.infv2_attn_path(0, 0) == tb.PATH_DENSE
    assert lib.infv2_attn_path(1, 0) == tb.PATH_SPARSE
    assert lib.infv2_attn_path(8192, -1) == tb.PATH_SPARSE


@no_gpu
def test_selection_and_switch_take_up_to_4064_blocks():
    lib = tb.load_library()

    def sel(S_k, S_q=10, stride=0, **kw):
        a = dict(q=FAKE, kc=FAKE, idx=FAKE, B=1, H_q=32, H_kv=2, topk=64)
        a.update(kw)
        if stride:
            return lib.infv2_select_blocks_strided_lse(a["q"], a["kc"], a["idx"], None, a["B"], a["H_q"], a["H_kv"],
                                                       S_q, S_k, 128, 64, a["topk"], 1, 2, 0.0, stride, None)
        return lib.infv2_select_blocks(a["q"], a["kc"], a["idx"], None, a["B"], a["H_q"], a["H_kv"], S_q, S_k, 128,
                                       64, a["topk"], 1, 2, 0.0, None)
    # 4064 blocks pass the shape checks (and then stop at the missing output); 4065 do not
    assert sel(4064 * 64, idx=None) == tb.ERR_INVALID
    assert sel(4064 * 64 + 1) == tb.ERR_UNSUPPORTED
    assert sel(4064 * 64, stride=4, idx=None) == tb.ERR_INVALID
    assert sel(4064 * 64 + 1, stride=4) == tb.ERR_UNSUPPORTED

    def switch(S_k, ws=None, wsb=0):
        return lib.infv2_attn_fwd(FAKE, FAKE, FAKE, FAKE, None, None, 1, 32, 2, 10, S_k, 128, 64, 64, 1, 2, 0.0, 0,
                                  ws, wsb, None)
    assert switch(4064 * 64) == tb.ERR_WORKSPACE
    assert switch(4064 * 64 + 1) == tb.ERR_UNSUPPORTED
