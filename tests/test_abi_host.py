"""C ABI checks that need no GPU: exports, blob layout, host packer round
trip, and argument validation (which returns before anything is enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest

import int4_group_quantized_moe_amd as moe
from int4_group_quantized_moe_amd import _ffi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_sources():
    import glob
    return [open(f).read() for f in sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))]


def header_functions():
    names = set()
    for src in header_sources():
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 12
    h = moe.lib()
    for n in names:
        assert hasattr(h, n), n
        assert n in _ffi.exported_symbols(), n


def test_boundary_names():
    """The boundary exports the calls the layer's C ABI is specified with:
    router + top-k, experts with a given routing, the whole layer, the chain
    step around it (residual add + RMSNorm), layout, packer and workspace."""
    names = set(header_functions())
    for n in ("moe_router_topk", "moe_experts_forward", "moe_layer_forward",
              "moe_residual_rmsnorm", "moe_blob_layout", "moe_pack_expert",
              "moe_workspace_bytes", "moe_status_string", "moe_version", "moe_chain_forward",
              "moe_chain_status", "moe_dense_layout", "moe_pack_dense"):
        assert n in names, n


def test_every_export_cites_its_passage():
    """Each declaration's comment names the passage of the pages that defines
    it, or says that it is not on the pages."""
    src = "\n".join(header_sources())
    for n in header_functions():
        m = re.search(r"/\*((?:(?!\*/).)*?)\*/\s*(?:const char\*|int|size_t|int32_t|void)\s+" + n + r"\s*\(",
                      src, flags=re.S)
        assert m, n
        doc = m.group(1)
        assert ("Defined by" in doc or "Not a passage" in doc or "Pure host function" in doc
                or "same call as" in doc or "for callers that cannot" in doc), n


def test_chain_status_word_inside_workspace():
    for T in (1, 4, 64):
        d = moe.make_desc(T, 2048, 512, 10, 512, 512)
        ws = np.zeros(moe.moe_workspace_bytes(d), np.uint8)
        addr = moe.moe_chain_status(d, ws)
        off = addr - ws.ctypes.data
        assert 0 <= off and off + 4 <= ws.nbytes and off % 4 == 0
        pi, _, _ = moe.moe_workspace_routing(d, ws)
        assert pi != addr


def test_host_code_under_sanitizers(tmp_path):
    """host.cpp (validation, blob layout, workspace plan, host packer) built
    with g++ under the address and undefined-behaviour sanitizers and driven
    through its C ABI by tests/sanitize/host_checks.cpp."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    csrc = os.path.join(ROOT, "int4_group_quantized_moe_amd", "csrc")
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-static-libasan",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", csrc, os.path.join(csrc, "host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                                UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks passed" in r.stdout


def test_version_and_status_strings():
    assert moe.moe_version().startswith("moe-gfx950")
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert moe.moe_status_string(st) != "unknown status"
    assert moe.moe_status_string(-99) == "unknown status"


@pytest.mark.parametrize("bits,H,I,expect", [
    (4, 2048, 512, 1769472),     # 3 x 524288 code bytes + 3 x 65536 scale/bias bytes
    (8, 2048, 512, 3342336),
    (4, 256, 128, 55296),
])
def test_blob_sizes(bits, H, I, expect):
    d = moe.make_desc(1, H, 16, 2, I, I, bits=bits)
    L = moe.moe_blob_layout(d, I)
    assert L.blob_bytes == expect
    assert L.blob_bytes % 256 == 0 and L.shared_bytes % 256 == 0
    assert L.shared_gate_offset >= L.blob_bytes
    assert L.shared_bytes >= L.shared_gate_offset + 4 * H
    assert L.row_tile == 16 and L.kblock_cols == (128 if bits == 4 else 64)


def unpack_blob(blob: np.ndarray, bits: int, H: int, I: int, L):
    """Reads the documented blob layout back into logical arrays."""
    kbc = L.kblock_cols
    gpk = L.groups_per_kblock

    def section(off, rows, cols, nmat, unit, tile):
        qs = [np.zeros((rows, cols), np.uint8) for _ in range(nmat)]
        sbs = [np.zeros((2, rows, cols // 64), np.uint16) for _ in range(nmat)]
        for t in range(rows // 16):
            for kb in range(cols // kbc):
                u = off + t * tile + kb * unit
                for m in range(nmat):
                    codes = blob[u + m * 1024: u + (m + 1) * 1024].reshape(16, 64)
                    for rl in range(16):
                        row = codes[rl]
                        if bits == 4:
                            vals = np.empty(128, np.uint8)
                            vals[0::2] = row & 15
                            vals[1::2] = row >> 4
                        else:
                            vals = row
                        qs[m][t * 16 + rl, kb * kbc:(kb + 1) * kbc] = vals
                    sb = blob[u + nmat * 1024 + m * 16 * gpk * 4:
                              u + nmat * 1024 + (m + 1) * 16 * gpk * 4].view(np.uint16)
                    sb = sb.reshape(16, gpk, 2)
                    for rl in range(16):
                        for gi in range(gpk):
                            sbs[m][0, t * 16 + rl, kb * gpk + gi] = sb[rl, gi, 0]
                            sbs[m][1, t * 16 + rl, kb * gpk + gi] = sb[rl, gi, 1]
        return qs, sbs

    (qg, qu), (sg, su) = section(L.gu_offset, I, H, 2, L.gu_unit_bytes, L.gu_tile_bytes)
    (qd,), (sd,) = section(L.down_offset, H, I, 1, L.down_unit_bytes, L.down_tile_bytes)
    return qg, qu, qd, sg, su, sd


@pytest.mark.parametrize("bits", [4, 8])
def test_host_packer_round_trip(bits):
    rng = np.random.default_rng(7)
    H, I = 256, 128
    d = moe.make_desc(1, H, 4, 2, I, I, bits=bits)
    L = moe.moe_blob_layout(d, I)
    qg = rng.integers(0, 1 << bits, (I, H)).astype(np.uint8)
    qu = rng.integers(0, 1 << bits, (I, H)).astype(np.uint8)
    qd = rng.integers(0, 1 << bits, (H, I)).astype(np.uint8)
    sg = rng.integers(0, 65536, (2, I, H // 64)).astype(np.uint16)
    su = rng.integers(0, 65536, (2, I, H // 64)).astype(np.uint16)
    sd = rng.integers(0, 65536, (2, H, I // 64)).astype(np.uint16)
    wsg = rng.standard_normal(H).astype(np.float32)
    blob = np.full(L.shared_bytes, 0xAB, np.uint8)
    moe.moe_pack_expert(d, I, qg, qu, qd, sg, su, sd, wsg, blob)
    got = unpack_blob(blob, bits, H, I, L)
    for a, b in zip(got, (qg, qu, qd, sg, su, sd)):
        assert np.array_equal(a, b)
    off = L.shared_gate_offset
    assert np.array_equal(blob[off:off + 4 * H].view(np.float32), wsg)
    # padding between sections is zero
    end = L.down_offset + (H // 16) * L.down_tile_bytes
    assert np.all(blob[end:L.blob_bytes] == 0)


@pytest.mark.parametrize("H,E,shared", [(256, 16, True), (2048, 512, True), (128, 3, False)])
def test_dense_packer_layout(H, E, shared):
    """moe_pack_dense writes the documented dense-blob format: codes row after
    row, value 2j in the low nibble of byte j; then one (scale, bias) word per
    row and group from words_offset; rows = E (+1 for the shared gate)."""
    rng = np.random.default_rng(11)
    d = moe.make_desc(1, H, E, 2, 128, 128, shared=shared, dense_q4=True)
    L = moe.moe_dense_layout(d)
    R, G = E + (1 if shared else 0), H // 64
    assert L.rows == R and L.words_offset % 256 == 0 and L.bytes % 256 == 0
    assert L.words_offset >= R * H // 2 and L.bytes >= L.words_offset + 4 * R * G
    q = rng.integers(0, 16, (R, H)).astype(np.uint8)
    sb = rng.integers(0, 65536, (2, R, G)).astype(np.uint16)
    blob = np.full(L.bytes, 0xAB, np.uint8)
    moe.moe_pack_dense(d, q, sb, blob)
    codes = blob[:R * H // 2].reshape(R, H // 2)
    assert np.array_equal(codes & 15, q[:, 0::2]) and np.array_equal(codes >> 4, q[:, 1::2])
    words = blob[L.words_offset:L.words_offset + 4 * R * G].view(np.uint32).reshape(R, G)
    assert np.array_equal(words & 0xFFFF, sb[0]) and np.array_equal(words >> 16, sb[1])
    assert np.all(blob[R * H // 2:L.words_offset] == 0)
    assert np.all(blob[L.words_offset + 4 * R * G:] == 0)
    bad = q.copy()
    bad[0, 1] = 16
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_dense(d, bad, sb, blob)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_host_packer_rejects_out_of_range_codes():
    H, I = 256, 128
    d = moe.make_desc(1, H, 4, 2, I, I, bits=4)
    z = np.zeros((I, H), np.uint8)
    bad = z.copy()
    bad[3, 5] = 16
    sb = np.zeros((2, I, H // 64), np.uint16)
    sbd = np.zeros((2, H, I // 64), np.uint16)
    blob = np.zeros(moe.moe_blob_layout(d, I).blob_bytes, np.uint8)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_expert(d, I, bad, z, z.T.copy(), sb, sb, sbd, None, blob)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# validation: every one of these returns before any device call

FAKE = 1 << 30          # 256-aligned fake address; never dereferenced


def _layer(d, x=FAKE, rw=FAKE, rb=None, slab=FAKE, st=FAKE, sh=FAKE, out=FAKE, ws=FAKE):
    return moe.lib().moe_layer_forward(ctypes.byref(d), x, rw, rb, slab, st, sh, out, ws, None)


@pytest.mark.parametrize("mut,status", [
    (dict(bits=5), moe.MOE_ERR_UNSUPPORTED),
    (dict(group=32), moe.MOE_ERR_UNSUPPORTED),
    (dict(top_k=17), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=4, top_k=5), moe.MOE_ERR_INVALID_ARG),
    (dict(hidden=200), moe.MOE_ERR_UNSUPPORTED),
    (dict(inter=100), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=7), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_tokens=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(flags=8), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_stride=1769472 + 100), moe.MOE_ERR_MISALIGNED),
    (dict(expert_stride=1024), moe.MOE_ERR_MISALIGNED),
])
def test_desc_validation(mut, status):
    d = moe.make_desc(1, 2048, 256, 8, 512, 512)
    for k, v in mut.items():
        setattr(d, k, v)
    assert _layer(d) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), moe.MOE_ERR_INVALID_ARG),
    (dict(x=FAKE + 2), moe.MOE_ERR_MISALIGNED),
    (dict(rw=None), moe.MOE_ERR_INVALID_ARG),
    (dict(slab=FAKE + 64), moe.MOE_ERR_MISALIGNED),
    (dict(st=None), moe.MOE_ERR_INVALID_ARG),
    (dict(sh=None), moe.MOE_ERR_INVALID_ARG),
    (dict(out=None), moe.MOE_ERR_INVALID_ARG),
    (dict(ws=FAKE + 16), moe.MOE_ERR_MISALIGNED),
])
def test_pointer_validation(kw, status):
    d = moe.make_desc(1, 2048, 256, 8, 512, 512)
    assert _layer(d, **kw) == status


def test_router_bias_required_when_flagged():
    d = moe.make_desc(64, 2048, 512, 10, 512, 512, router_bias=True)
    assert _layer(d, rb=None) == moe.MOE_ERR_INVALID_ARG


def test_zero_tokens_is_a_no_op():
    d = moe.make_desc(0, 2048, 256, 8, 512, 512)
    assert _layer(d) == moe.MOE_OK


def test_other_entry_points_validate():
    d = moe.make_desc(1, 2048, 256, 8, 512, 512)
    h = moe.lib()
    bad = moe.make_desc(1, 2048, 256, 8, 512, 512)
    bad.bits = 3
    assert h.moe_router_topk(ctypes.byref(bad), FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE,
                             None) == moe.MOE_ERR_UNSUPPORTED
    assert h.moe_router_topk(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE,
                             None) == moe.MOE_ERR_INVALID_ARG   # gamma without w_sg
    assert h.moe_experts_forward(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, None) == moe.MOE_ERR_INVALID_ARG  # shared gate missing
    assert h.moe_rmsnorm(ctypes.byref(d), None, None, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert h.moe_chain_forward(ctypes.byref(d), 0, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 21,
                               FAKE, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert h.moe_chain_forward(ctypes.byref(d), 2, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1000,
                               FAKE, FAKE, FAKE, None) == moe.MOE_ERR_MISALIGNED
    assert moe.moe_workspace_bytes(bad) == 0
    assert moe.moe_workspace_bytes(d) > 0


def test_valid_call_without_device_reports_no_device():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: fake pointers must not reach a launch")
    d = moe.make_desc(1, 2048, 256, 8, 512, 512)
    assert _layer(d) == moe.MOE_ERR_NO_DEVICE
