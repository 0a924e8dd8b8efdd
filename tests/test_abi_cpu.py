"""The C ABI library loads and exports every symbol include/bitlinear.h declares; host-only
helpers and argument validation behave as documented.  No compute call reaches a GPU:
every call here is rejected on the host before anything is enqueued."""
import ctypes
import os
import re
import subprocess

import pytest

import bitlinear_fwd_amd as bl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def test_library_present():
    assert os.path.exists(bl.LIB_PATH), "build with `python -m bitlinear_fwd_amd.build`"


def test_library_loads_without_unresolved_symbols():
    # dlopen with immediate binding: every referenced symbol (kernel launch stubs
    # included) must resolve
    out = subprocess.run(["nm", "-D", "--undefined-only", bl.LIB_PATH], capture_output=True, text=True).stdout
    assert "__device_stub__" not in out, out
    ctypes.CDLL(bl.LIB_PATH, mode=os.RTLD_NOW)


def test_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(bl.EXPORTED_SYMBOLS)
    L = bl.lib()
    for name in declared:
        assert hasattr(L, name), name
    # and they are real dynamic symbols of the shared object
    out = subprocess.run(["nm", "-D", "--defined-only", bl.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_host_size_helpers():
    assert bl.n_pad(1) == 16 and bl.n_pad(16) == 16 and bl.n_pad(17) == 32
    assert bl.k_pad(1) == 256 and bl.k_pad(256) == 256 and bl.k_pad(257) == 512
    assert bl.packed_bytes(28672, 8192) == 58_720_256
    assert bl.packed_bytes(6912, 2560) == 4_423_680
    assert bl.packed_bytes(17, 300) == 32 * 512 // 4
    assert bl.packed_bytes(0, 5) == -1 and bl.k_pad(0) == -1
    assert bl.wq_workspace_bytes(100, 100) >= 256 * 8 + 4
    assert bl.version() >= 10000


def test_status_strings():
    for s in (bl.BL_OK, bl.BL_ERR_INVALID_ARG, bl.BL_ERR_UNSUPPORTED, bl.BL_ERR_HIP, 7):
        assert isinstance(bl.status_string(s), str) and bl.status_string(s)


FAKE = 0x10000  # 64 KiB-aligned non-null address; never dereferenced (calls are rejected first)


def test_forward_argument_validation():
    L = bl.lib()
    ok = dict(packed=FAKE, gamma=FAKE, xq=FAKE, a=FAKE, M=1, N=16, K=256, y=FAKE, acc=None)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return L.bitlinear_forward(d["packed"], d["gamma"], d["xq"], d["a"], d["M"], d["N"], d["K"], d["y"],
                                   d["acc"], None)

    assert call(packed=None) == bl.BL_ERR_INVALID_ARG
    assert call(gamma=None) == bl.BL_ERR_INVALID_ARG
    assert call(xq=None) == bl.BL_ERR_INVALID_ARG
    assert call(a=None) == bl.BL_ERR_INVALID_ARG
    assert call(y=None, acc=None) == bl.BL_ERR_INVALID_ARG
    assert call(M=0) == bl.BL_ERR_INVALID_ARG
    assert call(N=0) == bl.BL_ERR_INVALID_ARG
    assert call(K=-3) == bl.BL_ERR_INVALID_ARG
    assert call(K=(1 << 24) + 1) == bl.BL_ERR_INVALID_ARG
    assert call(packed=FAKE + 8) == bl.BL_ERR_INVALID_ARG  # packed must be 16-byte aligned
    assert call(xq=FAKE + 4) == bl.BL_ERR_INVALID_ARG
    assert call(y=FAKE + 2) == bl.BL_ERR_INVALID_ARG


def test_quantize_argument_validation():
    L = bl.lib()
    ws = bl.wq_workspace_bytes(16, 256)
    assert L.bitlinear_quantize_weights(None, 16, 256, FAKE, FAKE, FAKE, ws, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_weights(FAKE, 16, 256, FAKE, FAKE, FAKE, ws - 1, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_weights(FAKE, 0, 256, FAKE, FAKE, FAKE, ws, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_weights(FAKE, 16, 256, FAKE + 4, FAKE, FAKE, ws, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_weights(FAKE, 1 << 21, 1 << 20, FAKE, FAKE, FAKE, ws, None) == bl.BL_ERR_UNSUPPORTED
    assert L.bitlinear_quantize_acts(FAKE, 5, 1, 16, FAKE, FAKE, None, None) == bl.BL_ERR_UNSUPPORTED
    assert L.bitlinear_quantize_acts(None, bl.BL_F32, 1, 16, FAKE, FAKE, None, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_acts(FAKE, bl.BL_F32, 0, 16, FAKE, FAKE, None, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_acts(FAKE + 2, bl.BL_F32, 1, 16, FAKE, FAKE, None, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_acts(FAKE, bl.BL_BF16, 1, 16, FAKE + 8, FAKE, None, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_quantize_acts(FAKE, bl.BL_BF16, 1, 16, FAKE, FAKE, FAKE + 2, None) == bl.BL_ERR_INVALID_ARG


def test_binding_rejects_cpu_tensors():
    import torch

    with pytest.raises(ValueError):
        bl.quantize_weights(torch.zeros(4, 4))
    with pytest.raises(ValueError):
        bl.quantize_acts(torch.zeros(4, 4))


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "bitlinear_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "liboracle" not in src and "bitlinear_oracle" not in src, f


def test_grouped_argument_validation():
    L = bl.lib()
    one = (bl.BlMatrix * 9)(*[bl.BlMatrix(FAKE, FAKE, 16, FAKE, None) for _ in range(9)])
    addr = ctypes.addressof(one)
    ok = dict(mats=addr, count=2, x=FAKE, dt=bl.BL_BF16, M=1, K=256, xq=FAKE, a=FAKE)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return L.bitlinear_forward_grouped(d["mats"], d["count"], d["x"], d["dt"], d["M"], d["K"], d["xq"], d["a"],
                                           None)

    assert call(mats=None) == bl.BL_ERR_INVALID_ARG
    assert call(count=0) == bl.BL_ERR_INVALID_ARG
    assert call(count=9) == bl.BL_ERR_INVALID_ARG
    assert call(x=None) == bl.BL_ERR_INVALID_ARG
    assert call(M=0) == bl.BL_ERR_INVALID_ARG
    assert call(K=(1 << 24) + 1) == bl.BL_ERR_INVALID_ARG
    assert call(dt=7) == bl.BL_ERR_UNSUPPORTED
    assert call(xq=FAKE + 4) == bl.BL_ERR_INVALID_ARG
    bad = (bl.BlMatrix * 2)(bl.BlMatrix(FAKE, FAKE, 16, FAKE, None), bl.BlMatrix(FAKE + 8, FAKE, 16, FAKE, None))
    assert call(mats=ctypes.addressof(bad)) == bl.BL_ERR_INVALID_ARG  # misaligned packed
    bad[1] = bl.BlMatrix(FAKE, FAKE, 0, FAKE, None)
    assert call(mats=ctypes.addressof(bad)) == bl.BL_ERR_INVALID_ARG  # N = 0
    bad[1] = bl.BlMatrix(FAKE, FAKE, 16, None, None)
    assert call(mats=ctypes.addressof(bad)) == bl.BL_ERR_INVALID_ARG  # no output


def test_probe_argument_validation():
    L = bl.lib()
    assert L.bitlinear_probe_stream_words(1024) == 1
    assert L.bitlinear_probe_stream_words(32768) == 1 and L.bitlinear_probe_stream_words(32769 * 1024) == 1025
    assert L.bitlinear_probe_stream_words(1000) == -1 and L.bitlinear_probe_stream_words(0) == -1
    assert L.bitlinear_probe_stream(None, 1024, FAKE, 1, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_probe_stream(FAKE, 1000, FAKE, 1, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_probe_stream(FAKE + 8, 1024, FAKE, 1, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_probe_stream(FAKE, 65536, FAKE, 1, None) == bl.BL_ERR_INVALID_ARG  # needs 2 words
    assert L.bitlinear_probe_mfma(0, 1, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_probe_mfma(1, 0, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_probe_mfma(1, 1, None, None) == bl.BL_ERR_INVALID_ARG


def test_subln_argument_validation():
    L = bl.lib()
    nan, inf = float("nan"), float("inf")
    q = L.bitlinear_subln_quantize_acts
    assert q(None, bl.BL_F32, 1, 16, None, 1e-5, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert q(FAKE, bl.BL_F32, 1, 16, None, -1e-5, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert q(FAKE, bl.BL_F32, 1, 16, None, nan, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert q(FAKE, bl.BL_F32, 1, 16, None, inf, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert q(FAKE, bl.BL_F32, 1, 16, FAKE + 2, 1e-5, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG  # gain alignment
    assert q(FAKE, bl.BL_F32, 0, 16, None, 1e-5, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert q(FAKE, 9, 1, 16, None, 1e-5, FAKE, FAKE, None) == bl.BL_ERR_UNSUPPORTED
    assert q(FAKE, bl.BL_BF16, 1, 16, None, 1e-5, FAKE + 8, FAKE, None) == bl.BL_ERR_INVALID_ARG
    f = L.bitlinear_forward_subln
    ok = dict(packed=FAKE, gamma=FAKE, x=FAKE, dt=bl.BL_BF16, M=1, N=16, K=256, gain=None, eps=1e-5, y=FAKE,
              acc=None, xq=FAKE, sc=FAKE)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return f(d["packed"], d["gamma"], d["x"], d["dt"], d["M"], d["N"], d["K"], d["gain"], d["eps"], d["y"],
                 d["acc"], d["xq"], d["sc"], None)

    assert call(packed=None) == bl.BL_ERR_INVALID_ARG
    assert call(sc=None) == bl.BL_ERR_INVALID_ARG
    assert call(y=None, acc=None) == bl.BL_ERR_INVALID_ARG
    assert call(eps=-1.0) == bl.BL_ERR_INVALID_ARG
    assert call(gain=FAKE + 1) == bl.BL_ERR_INVALID_ARG
    assert call(K=(1 << 24) + 1) == bl.BL_ERR_INVALID_ARG
    assert call(dt=3) == bl.BL_ERR_UNSUPPORTED
    one = (bl.BlMatrix * 2)(*[bl.BlMatrix(FAKE, FAKE, 16, FAKE, None) for _ in range(2)])
    g = L.bitlinear_forward_grouped_subln
    assert g(ctypes.addressof(one), 2, FAKE, bl.BL_BF16, 1, 256, None, nan, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert g(ctypes.addressof(one), 0, FAKE, bl.BL_BF16, 1, 256, None, 0.0, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG
    assert g(None, 2, FAKE, bl.BL_BF16, 1, 256, None, 0.0, FAKE, FAKE, None) == bl.BL_ERR_INVALID_ARG


def test_subln_plan_host():
    # one launch for the decode shapes of a 2B-class layer; beyond the register budget
    # (fp32, long rows) the two-kernel path; prefill sizes use the prefill plan
    assert bl.forward_subln_plan(1, 6912, 2560)["kernel"] == "fused"
    assert bl.forward_subln_plan(1, 2560, 6912)["kernel"] == "fused"
    assert bl.forward_subln_plan(4, 640, 2560)["kernel"] == "fused"
    assert bl.forward_subln_plan(1, 700, 28672, "f32")["kernel"] == "decode"
    assert bl.forward_subln_plan(8, 700, 2560)["kernel"] == "decode"
    assert bl.forward_subln_plan(2048, 6912, 2560)["kernel"] == "prefill"
    # the plain fused plans are unchanged by the normalising form
    assert bl.forward_fused_plan(3, 65600, 768, "f32")["acts"] == "lds"


def test_gated_relu2_argument_validation():
    L = bl.lib()
    f = L.bitlinear_forward_gated_relu2
    ok = dict(gp=FAKE, gg=FAKE, up=FAKE, ug=FAKE, x=FAKE, dt=bl.BL_BF16, M=1, N=16, K=256, subln=0, gain=None,
              eps=0.0, h=FAKE, xq=FAKE, sc=FAKE, ws=None, wsb=0)

    def call(**kw):
        d = dict(ok)
        d.update(kw)
        return f(d["gp"], d["gg"], d["up"], d["ug"], d["x"], d["dt"], d["M"], d["N"], d["K"], d["subln"], d["gain"],
                 d["eps"], d["h"], d["xq"], d["sc"], d["ws"], d["wsb"], None)

    assert call(gp=None) == bl.BL_ERR_INVALID_ARG
    assert call(ug=None) == bl.BL_ERR_INVALID_ARG
    assert call(h=None) == bl.BL_ERR_INVALID_ARG
    assert call(up=FAKE + 4) == bl.BL_ERR_INVALID_ARG
    assert call(subln=2) == bl.BL_ERR_INVALID_ARG
    assert call(subln=1, eps=-1.0) == bl.BL_ERR_INVALID_ARG
    assert call(dt=5) == bl.BL_ERR_UNSUPPORTED
    # off the one-kernel path (M = 8) the workspace is required
    assert call(M=8) == bl.BL_ERR_INVALID_ARG
    assert call(M=8, ws=FAKE, wsb=8 * 16 * 4 - 1) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_gated_relu2_workspace_bytes(8, 16) == 512
    assert L.bitlinear_gated_relu2_workspace_bytes(0, 16) == -1
    assert bl.forward_gated_relu2_plan(1, 6912, 2560)["kernel"] == "fused"
    assert bl.forward_gated_relu2_plan(8, 6912, 2560)["kernel"] == "decode"


def test_lut_plan_and_validation():
    L = bl.lib()
    assert bl.forward_lut_plan(1, 6912, 2560)["kernel"] == "lut"
    assert bl.forward_lut_plan(5, 64, 256) is None
    assert bl.forward_lut_plan(1, 64, 28672) is None
    assert L.bitlinear_forward_lut(None, FAKE, FAKE, FAKE, 1, 16, 256, FAKE, None, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_forward_lut(FAKE, FAKE, FAKE, FAKE, 1, 16, 256, None, None, None) == bl.BL_ERR_INVALID_ARG
    assert L.bitlinear_forward_lut(FAKE, FAKE, FAKE, FAKE, 5, 16, 256, FAKE, None, None) == bl.BL_ERR_UNSUPPORTED


def test_binary_sizes_plan_and_validation():
    L = bl.lib()
    assert bl.kb_pad(6912) == 7168 and bl.kb_pad(512) == 512 and L.bitlinear_kb_pad(0) == -1
    assert bl.packed_bytes_binary(28672, 8192) == 28672 * 8192 // 8
    assert bl.packed_bytes_binary(17, 300) == 32 * 512 // 8
    assert bl.forward_binary_plan(1, 6912, 2560)["kernel"] == "binary"
    assert bl.forward_binary_plan(5, 64, 512) is None
    ws = bl.wq_workspace_bytes(16, 512)
    q = L.bitlinear_quantize_weights_binary
    assert q(None, 16, 512, FAKE, FAKE, FAKE, ws, None) == bl.BL_ERR_INVALID_ARG
    assert q(FAKE, 16, 512, FAKE + 8, FAKE, FAKE, ws, None) == bl.BL_ERR_INVALID_ARG
    assert q(FAKE, 16, 512, FAKE, FAKE, FAKE, ws - 1, None) == bl.BL_ERR_INVALID_ARG
    f = L.bitlinear_forward_binary
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 16, 512, None, None, None) == bl.BL_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 5, 16, 512, FAKE, None, None) == bl.BL_ERR_UNSUPPORTED


def test_token_group_routing():
    # 17..64 tokens go to the decode kernel with token groups where its L2 re-reads of the
    # token rows cost less than the prefill kernel's K loop; 65 and more always prefill
    # (m, n, k, row blocks per workgroup)
    decode = [(17, 2560, 2560, 1), (64, 2560, 2560, 1), (48, 6912, 2560, 2), (64, 2560, 6912, 1),
              (17, 8192, 28672, 2), (48, 8192, 28672, 2), (17, 28672, 8192, 4), (32, 28672, 8192, 4),
              (17, 28672, 4096, 4), (40, 72, 700, 1)]
    prefill = [(48, 28672, 8192), (64, 28672, 8192), (48, 30000, 512), (64, 24000, 1024), (65, 64, 256)]
    for m, n, k, rb in decode:
        p = bl.forward_plan(m, n, k)
        assert p["kernel"] == "decode" and p["row_blocks"] == rb, (m, n, k, p)
        assert (p["threads"] // 64) * rb * ((m + 15) // 16) <= 32, (m, n, k, p)
    for m, n, k in prefill:
        assert bl.forward_plan(m, n, k)["kernel"] == "prefill", (m, n, k)


def test_prefill_plans():
    # host-only sweep of the prefill planner: a supported tile shape, 256 threads per K group
    # (512 for the eight-wave 64 x 384 tile, one K group), and a grid of whole XCD rounds
    # covering every 64-row tile
    for m in (17, 65, 100, 333, 1000, 1536, 2048, 4096, 8192):
        for n in (1, 16, 640, 2000, 2560, 6912, 8192, 28672):
            for k in (1, 256, 2560, 6912, 28672):
                p = bl.forward_plan(m, n, k)
                if p["kernel"] != "prefill":
                    assert m <= 64, (m, n, k, p)
                    continue
                assert p["tile_m"] == 64 and p["tile_n"] in (192, 256, 384), (m, n, k, p)
                assert p["k_groups"] in (1, 2), (m, n, k, p)
                if p["tile_n"] == 384:
                    assert p["k_groups"] == 1 and p["threads"] == 512 and n >= 384, (m, n, k, p)
                else:
                    assert p["threads"] == 256 * p["k_groups"], (m, n, k, p)
                tiles = -(-m // 64) * -(-n // p["tile_n"])
                assert p["workgroups"] == 8 * -(-tiles // 8), (m, n, k, p)
                if p["k_groups"] == 2:
                    assert tiles <= 512, (m, n, k, p)


def test_split_tail_plans_cover_every_tile_once():
    # host-only sweep of the workspace planner (bitlinear_forward_ws): where it splits a tail,
    # the blocks of the grid must cover every output tile exactly once, whole tiles by one
    # block and each tail tile by K ranges that partition its 256-column chunks, with the
    # workspace large enough for the counters and every range's partial tile.  The block ->
    # work map below is the one the kernel documents: block b < rounds x slots takes whole
    # tile (b % 8) x (rounds x slots / 8) + b / 8; block b past them, with s = (b - D) / 8,
    # takes range s % parts of tail tile 8 (s / parts) + b % 8 (none when that is >= tail).
    seen_split = 0
    for m in (65, 333, 614, 1000, 1037, 1061, 1345, 1536, 1571, 1600, 2048, 2098, 2961, 3000, 3074, 4096, 4721, 4904,
              8192):
        for n in (640, 2560, 2600, 4100, 6912, 8000, 8003, 9000, 10240, 12000, 19968, 28672):
            for k in (256, 700, 1000, 2560, 3001, 6912, 8192):
                p = bl.forward_ws_plan(m, n, k)
                nbytes = bl.forward_ws_bytes(m, n, k)
                if not p.get("split_tail"):
                    assert nbytes == 0 and p == bl.forward_plan(m, n, k), (m, n, k, p)
                    continue
                seen_split += 1
                assert p["tile_n"] == bl.forward_plan(m, n, k)["tile_n"] and nbytes <= 8 << 20, (m, n, k, p)
                bn, chunks = p["tile_n"], bl.k_pad(k) // 256
                tiles = -(-m // 64) * -(-n // bn)
                slots = 256 * (3 if bn == 256 else 4)
                rounds, tail, parts, cpp = p["rounds"], p["split_tiles"], p["k_ranges"], p["chunks_per_range"]
                assert p["tile_m"] == 64 and p["threads"] == 256 and p["k_groups"] == 1, p
                assert rounds == tiles // slots and tail == tiles - rounds * slots and 0 < tail < slots, (m, n, k, p)
                assert parts >= 2 and (parts - 1) * cpp < chunks <= parts * cpp, (m, n, k, p)
                assert nbytes == tail * parts * 64 * bn * 4, (m, n, k, p, nbytes)
                dp = rounds * slots
                assert dp % 8 == 0 and p["workgroups"] == dp + 8 * parts * -(-tail // 8), (m, n, k, p)
                whole = [0] * tiles
                ranges = {}
                for b in range(p["workgroups"]):
                    if b < dp:
                        whole[(b % 8) * (dp // 8) + b // 8] += 1
                        continue
                    s_ = (b - dp) // 8
                    i = 8 * (s_ // parts) + b % 8
                    if i < tail:
                        ranges.setdefault(dp + i, []).append(s_ % parts)
                assert all(c == 1 for c in whole[:dp]) and not any(whole[dp:]), (m, n, k, p)
                assert sorted(ranges) == list(range(dp, tiles)), (m, n, k, p)
                for t, js in ranges.items():
                    assert sorted(js) == list(range(parts)), (m, n, k, t, js)
                    covered = sorted(c for j in js for c in range(j * cpp, min(chunks, (j + 1) * cpp)))
                    assert covered == list(range(chunks)), (m, n, k, t)
    assert seen_split > 20


def dt_of(name, p):
    # the 5..16-token LDS form reads bf16 x only
    return name == "fused bf16"


def test_launch_plans_cover_every_tile():
    # host-only sweep of every planner: a plan's waves x tiles per wave must cover all K
    # tiles, and its workgroups all row blocks, or outputs would silently go missing
    shapes_k = [1, 8, 255, 256, 257, 1000, 2560, 4096, 6912, 8192, 12000, 28672, 40000]
    shapes_n = [1, 16, 17, 640, 2560, 6912, 28672]
    for m in (1, 2, 3, 4, 5, 8, 16, 17, 32, 33, 48, 64):
        for k in shapes_k:
            chunks = bl.k_pad(k) // 256
            chunks_b = bl.kb_pad(k) // 512
            for n in shapes_n:
                rblocks = bl.n_pad(n) // 16
                plans = [("forward", bl.forward_plan(m, n, k))]
                for dt in ("bf16", "f32"):
                    plans.append(("fused " + dt, bl.forward_fused_plan(m, n, k, dt)))
                    plans.append(("subln", bl.forward_subln_plan(m, n, k, dt)))
                    plans.append(("gated", bl.forward_gated_relu2_plan(m, n, k, dt, True)))
                for name, p in plans:
                    assert p["workgroups"] >= 1 and p["threads"] % 64 == 0 and 64 <= p["threads"] <= 1024, (name, p)
                    if p["kernel"] in ("fused", "decode") and p.get("acts") == "registers":
                        waves = p["threads"] // 64
                        assert waves * p["tiles_per_wave"] >= chunks, (name, m, n, k, p)
                        assert waves <= 16 and (waves - 1) * p["tiles_per_wave"] < chunks, (name, m, n, k, p)
                        assert p["workgroups"] * p["row_blocks"] >= rblocks, (name, m, n, k, p)
                    if p["kernel"] == "fused" and p["acts"] == "lds16":
                        # 5..16 tokens, bf16, every workgroup quantises the input into LDS:
                        # eight waves of two token rows each, runs cover K
                        waves = p["threads"] // 64
                        assert 5 <= m <= 16 and dt_of(name, p) and k % 8 == 0 and k <= 7168 and m * k <= 65536, \
                            (name, m, n, k, p)
                        assert waves == 8 and waves * p["tiles_per_wave"] >= chunks, (name, m, n, k, p)
                        assert p["row_blocks"] * waves <= 32, (name, m, n, k, p)
                        assert p["workgroups"] * p["row_blocks"] >= rblocks, (name, m, n, k, p)
                    if p["kernel"] == "decode" and p["acts"] == "per-tile loads":
                        # waves split the K tiles into contiguous runs; workgroups own row blocks
                        assert p["threads"] // 64 <= (8 if m > 16 else 16), (name, m, n, k, p)
                        assert p["workgroups"] * p["row_blocks"] >= rblocks, (name, m, n, k, p)
                    assert p["kernel"] != "prefill" if m <= 16 else True, (name, m, n, k, p)
                lut = bl.forward_lut_plan(m, n, k)
                if lut is not None:
                    waves = lut["threads"] // 64
                    assert m <= 4 and waves * lut["tiles_per_wave"] >= chunks and lut["workgroups"] == rblocks
                    assert lut["lds_bytes"] == waves * lut["tiles_per_wave"] * m * 4352 <= 148 * 1024
                binp = bl.forward_binary_plan(m, n, k)
                if binp is not None:
                    waves = binp["threads"] // 64
                    assert m <= 4 and waves <= 16 and waves * binp["tiles_per_wave"] >= chunks_b
                    assert binp["workgroups"] == rblocks
