"""The C ABI library loads, exports every symbol include/awq.h declares, and
its host-side logic (validation, planning, sizes) behaves as documented.
No kernel is launched here: every call below fails validation or only plans."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    import weight_only_bit_awq_amd as awq
    if not os.path.exists(awq.LIB_PATH):
        from weight_only_bit_awq_amd import build
        build.build()
    return awq.library()


def declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(awq_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions([HEADER])
    for required in ("awq_pack", "awq_dequant", "awq_linear", "awq_unpack", "awq_pack_zeros",
                     "awq_linear_workspace_size", "awq_linear_workspace_bytes", "awq_qweight_words",
                     "awq_status_string"):
        assert required in names
    # the measurement aid has a header of its own
    assert "awq_stream_read" not in names
    assert "awq_stream_read" in declared_functions()


def test_every_declaration_cites_or_refers(lib):
    # each function of the layer's header is preceded by its own comment
    text = open(HEADER).read()
    body = text[text.index('extern "C" {'):]
    for name in declared_functions([HEADER]):
        pos = re.search(r"\b" + name + r"\s*\(", re.sub(r"/\*.*?\*/", lambda m: " " * len(m.group(0)), body,
                                                         flags=re.S)).start()
        before = body[:pos]
        assert "*/" in before[-1200:], f"{name}: no comment before its declaration"


def test_workspace_size(lib):
    import weight_only_bit_awq_amd as awq
    size_max = ctypes.c_size_t(-1).value
    for M, K, N in [(1, 4096, 4096), (512, 5120, 5120), (2048, 5120, 15360), (512, 13824, 5120)]:
        assert lib.awq_linear_workspace_size(M, K, N, 128) == awq.linear_workspace_bytes(M, K, N, 128)
    assert lib.awq_linear_workspace_size(512, 5120, 5120, 128) > 0
    assert lib.awq_linear_workspace_size(1, 4000, 16, 128) == size_max   # K % group
    assert lib.awq_linear_workspace_size(1, 480, 16, 96) == size_max     # group
    assert lib.awq_linear_workspace_size(0, 4096, 4096, 128) == 0


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_binding_covers_header(lib):
    import weight_only_bit_awq_amd as awq
    assert set(declared_functions()) <= set(awq._SIGS)


def test_status_strings_and_version(lib):
    assert lib.awq_status_string(0) == b"AWQ_OK"
    for code in range(-8, 0):
        assert lib.awq_status_string(code).startswith(b"AWQ_ERR")
    assert lib.awq_abi_version() == 1


def test_qweight_words(lib):
    import oracle
    for K, N in [(128, 16), (4096, 4096), (96, 24), (11008, 4096), (32, 8)]:
        assert lib.awq_qweight_words(K, N) == oracle.device_words(K, N)
    assert lib.awq_qweight_words(0, 16) == 0


def test_validation_errors_before_launch(lib):
    import weight_only_bit_awq_amd as awq
    sz = ctypes.c_size_t(0)
    # group must be 32, 64 or a multiple of 128
    assert lib.awq_linear_workspace_bytes(1, 480, 16, 96, ctypes.byref(sz)) == -3
    assert lib.awq_linear_workspace_bytes(1, 4096, 16, 0, ctypes.byref(sz)) == -3
    # K % group, N % 8, negative sizes
    assert lib.awq_linear_workspace_bytes(1, 4000, 16, 128, ctypes.byref(sz)) == -2
    assert lib.awq_linear_workspace_bytes(1, 4096, 12, 128, ctypes.byref(sz)) == -2
    assert lib.awq_linear_workspace_bytes(-1, 4096, 16, 128, ctypes.byref(sz)) == -2
    # null pointers
    assert lib.awq_pack(None, 128, 16, None, None) == -1
    assert lib.awq_unpack(None, 128, 16, None, None) == -1
    assert lib.awq_pack_zeros(None, 1, 16, None, None) == -1
    assert lib.awq_dequant(None, None, None, 128, 16, 128, None, None) == -1
    assert lib.awq_linear(None, None, None, None, 1, 128, 16, 128, None, None, 0, None) == -1
    # misaligned pointers are rejected before any launch
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1001)
    assert lib.awq_linear(odd, fake, fake, fake, 1, 128, 16, 128, fake, None, 0, None) == -4
    # empty calls succeed without touching pointers
    assert lib.awq_linear(None, None, None, None, 0, 128, 16, 128, None, None, 0, None) == 0
    assert lib.awq_pack(None, 0, 16, None, None) == 0
    # bad plans
    p = awq.Plan()
    p.path = 1
    assert lib.awq_linear_plan(65, 4096, 4096, 128, ctypes.byref(p)) == -7
    p = awq.Plan()
    p.path = 1
    p.waves = 3
    assert lib.awq_linear_plan(1, 4096, 4096, 128, ctypes.byref(p)) == -7
    p = awq.Plan()
    p.path, p.tpw = 1, 3
    assert lib.awq_linear_plan(1, 4096, 4096, 128, ctypes.byref(p)) == -7
    p = awq.Plan()
    p.path, p.x_stage = 1, 1  # staged activations need M <= 16
    assert lib.awq_linear_plan(32, 4096, 4096, 128, ctypes.byref(p)) == -7
    # a K split over workgroups on the decode path: streamed activations
    # only, at most 16, partials in the workspace (refused without it)
    p = awq.Plan()
    p.path, p.split_k, p.x_stage = 1, 4, 1
    need = ctypes.c_size_t(0)
    assert lib.awq_linear_workspace_bytes_ex(1, 4096, 4096, 128, ctypes.byref(p), ctypes.byref(need)) == -7
    assert lib.awq_linear_ex(fake, fake, fake, fake, 1, 4096, 4096, 128, fake, None, 0, ctypes.byref(p), None) == -7
    p = awq.Plan()
    p.path, p.split_k = 1, 17
    assert lib.awq_linear_workspace_bytes_ex(1, 4096, 4096, 128, ctypes.byref(p), ctypes.byref(need)) == -7
    p = awq.Plan()
    p.path, p.split_k = 1, 4
    assert lib.awq_linear_workspace_bytes_ex(8, 4096, 4096, 128, ctypes.byref(p), ctypes.byref(need)) == 0
    assert need.value == 4 * 8 * 4096 * 4
    assert awq.linear_plan(8, 4096, 4096, 128, {"path": 1, "split_k": 4})["x_stage"] == 2
    assert awq.linear_plan(8, 256, 4096, 128, {"path": 1, "split_k": 4})["split_k"] == 2  # two bands
    assert lib.awq_linear_ex(fake, fake, fake, fake, 8, 4096, 4096, 128, fake, None, 0, ctypes.byref(p), None) == -5
    assert lib.awq_linear_ex(fake, fake, fake, fake, 8, 4096, 4096, 128, ctypes.c_void_p(0x1002), fake, 1 << 30,
                             ctypes.byref(p), None) == -4
    # prefill split-K: at most 16; a split plan without its workspace is refused before any launch
    p = awq.Plan()
    p.path, p.split_k = 2, 17
    assert lib.awq_linear_plan(512, 5120, 5120, 128, ctypes.byref(p)) == -7
    p = awq.Plan()
    p.path, p.split_k = 2, 4
    assert lib.awq_linear_ex(fake, fake, fake, fake, 512, 5120, 5120, 128, fake, None, 0, ctypes.byref(p), None) == -5
    assert lib.awq_linear_ex(fake, fake, fake, fake, 512, 5120, 5120, 128, fake, fake, 16, ctypes.byref(p), None) == -5
    # its reduction stores four outputs at a time: y must be 8-byte aligned
    y2 = ctypes.c_void_p(0x1002)
    big = 4 * 512 * 5120 * 4
    assert lib.awq_linear_ex(fake, fake, fake, fake, 512, 5120, 5120, 128, y2, fake, big, ctypes.byref(p), None) == -4
    assert lib.awq_linear_silu_mul_ex(fake, fake, fake, fake, 2048, 5120, 27648, 128, y2, fake, 1 << 40, None, None,
                                      None, None) == -4


def test_plans(lib):
    import weight_only_bit_awq_amd as awq
    plan = awq.linear_plan(1, 4096, 4096, 128)
    assert plan["path"] == 1 and plan["split_k"] == 1 and plan["waves"] in (1, 2, 4, 8, 16)
    assert plan["x_stage"] == 1 and plan["tpw"] in (1, 2)
    assert awq.linear_plan(32, 4096, 4096, 128)["x_stage"] == 2
    assert awq.linear_plan(64, 4096, 4096, 128)["path"] == 1
    assert awq.linear_plan(65, 4096, 4096, 128)["path"] == 2
    assert awq.linear_plan(2048, 5120, 15360, 128)["path"] == 2
    # decode plans and well-filled prefill plans need no workspace
    assert awq.linear_workspace_bytes(1, 4096, 12288, 128, {"path": 1, "split_k": 1}) == 0
    assert awq.linear_workspace_bytes(2048, 5120, 15360, 128) == 0
    # a prefill layer with few output tiles is split over K: fp32 partials per split
    p512 = awq.linear_plan(512, 5120, 5120, 128)
    assert p512["path"] == 2 and p512["split_k"] > 1
    assert awq.linear_workspace_bytes(512, 5120, 5120, 128) == p512["split_k"] * 512 * 5120 * 4
    assert awq.linear_workspace_bytes(512, 5120, 5120, 128, {"path": 2, "tile": 2, "split_k": 3}) == 3 * 512 * 5120 * 4
    # never more splits than K steps (a 256-row layer has two 128-row steps)
    assert awq.linear_plan(512, 256, 5120, 128, {"path": 2, "tile": 2, "split_k": 8})["split_k"] == 2


def test_prefill_plans_measured_choices(lib):
    # the automatic prefill plans measured best on the LLaMA-2-13B layers
    # (host logic only): the fp16 GEMM's step time depends on how many CUs
    # are busy, so the 5120 x 5120 layer at M = 2048 (160 tiles) runs unsplit
    # and the down projection (K = 13824) in three ranges; the W4A8 GEMM keeps
    # its flat model (tile 2, three splits for the 5120 x 5120 layer at 512)
    import weight_only_bit_awq_amd as awq
    want = {(2048, 5120, 15360): 1, (2048, 5120, 5120): 1, (2048, 5120, 27648): 1, (2048, 13824, 5120): 3,
            (512, 5120, 15360): 2, (512, 5120, 27648): 1, (512, 13824, 5120): 6}
    for (M, K, N), split in want.items():
        p = awq.linear_plan(M, K, N, 128)
        assert (p["path"], p["tile"], p["split_k"]) == (2, 3, split), (M, K, N, p)
    assert awq.linear_plan(512, 5120, 5120, 128)["split_k"] in (5, 6)
    assert awq.linear_w4a8_plan(512, 5120, 5120, 128) == {"path": 2, "split_k": 3, "tile": 2}
    assert awq.linear_w4a8_plan(2048, 5120, 5120, 128)["split_k"] == 1
    assert awq.linear_w4a8_plan(2048, 13824, 5120, 128)["split_k"] == 3


def test_batched_decode_plans(lib):
    # the automatic choices measured on the LLaMA-3-8B layers (host logic only)
    import weight_only_bit_awq_amd as awq
    for K, N in [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096)]:
        p1 = awq.linear_plan(1, K, N, 128)
        assert p1["path"] == 1 and p1["x_stage"] == 1          # one row: staged activations
    # eight-wave workgroups that would need more than one round of wave slots: four
    assert awq.linear_plan(1, 4096, 22016, 128)["waves"] == 4   # 1376 tiles
    assert awq.linear_plan(1, 4096, 16384, 128)["waves"] == 8   # 1024 tiles: one round
    assert awq.linear_plan(1, 4544, 18176, 64)["waves"] == 8    # other group sizes: from ~1536 tiles
    # one row whose activations need sixteen staging waves, on a wide layer: streamed, eight waves
    p = awq.linear_plan(1, 59392, 14848, 128)
    assert (p["x_stage"], p["waves"], p["tpw"]) == (2, 8, 4)
    assert awq.linear_plan(1, 59392, 4096, 128)["waves"] == 16  # 256 tiles: staged with sixteen
    p = awq.linear_plan(8, 4096, 6144, 128)                     # 384 tiles: streamed, two tiles, eight waves
    assert (p["path"], p["x_stage"], p["tpw"], p["waves"]) == (1, 2, 2, 8)
    p = awq.linear_plan(16, 4096, 6144, 128)                    # from 16 rows: four waves
    assert (p["path"], p["x_stage"], p["tpw"], p["waves"]) == (1, 2, 2, 4)
    p = awq.linear_plan(8, 4096, 4096, 128)                     # 256 tiles, 8 rows: streamed, one tile
    assert (p["path"], p["x_stage"], p["tpw"], p["waves"]) == (1, 2, 1, 4)
    assert awq.linear_plan(4, 4096, 4096, 128)["x_stage"] == 1  # 4 rows: staged
    p = awq.linear_plan(16, 4096, 28672, 128)                   # 1792 tiles: four per workgroup
    assert (p["path"], p["x_stage"], p["tpw"], p["waves"]) == (1, 2, 4, 4)
    p = awq.linear_plan(32, 4096, 28672, 128)                   # above 16 rows, wide: slab, one tile per wave
    assert (p["path"], p["x_stage"], p["tpw"], p["waves"], p["split_k"]) == (1, 3, 1, 8, 1)
    p = awq.linear_plan(32, 4096, 28672, 32)                    # 32-row groups at 32 rows: two
    assert p["tpw"] == 2
    p = awq.linear_plan(4, 14336, 4096, 128)                    # 256 tiles: staged, sixteen waves
    assert (p["x_stage"], p["waves"]) == (1, 16)
    p = awq.linear_plan(32, 14336, 4096, 128)                   # long K, narrow, 32 rows: K split four ways
    assert (p["path"], p["x_stage"], p["tpw"], p["waves"], p["split_k"]) == (1, 2, 4, 8, 4)
    assert awq.linear_workspace_bytes(32, 14336, 4096, 128) == 4 * 32 * 4096 * 4
    assert awq.linear_plan(16, 14336, 4096, 128)["split_k"] == 4
    assert awq.linear_plan(8, 14336, 4096, 128)["split_k"] == 1
    assert awq.linear_plan(32, 4096, 4096, 128)["split_k"] == 1
    assert awq.linear_plan(48, 4096, 28672, 128)["path"] == 2   # wide layer above 32 rows: GEMM
    assert awq.linear_plan(48, 4096, 4096, 128)["path"] == 1
    with pytest.raises(awq.AWQError):                           # four tiles only with streamed activations
        awq.linear_plan(1, 4096, 4096, 128, {"path": 1, "tpw": 4, "x_stage": 1})
    with pytest.raises(awq.AWQError):                           # and at most 32 rows
        awq.linear_plan(40, 4096, 4096, 128, {"path": 1, "tpw": 2, "x_stage": 2})


def test_slab_plans(lib):
    # x_stage 3 (eight waves on the same bands, two-band activation slabs in
    # LDS): automatic on the largest 16-row layers and wide ones above 16
    # rows, K split to about one round of workgroups with >= 16 bands each
    import weight_only_bit_awq_amd as awq
    p = awq.linear_plan(16, 14848, 59392, 128)                  # Falcon-180B-shaped up
    assert (p["x_stage"], p["tpw"], p["waves"], p["split_k"]) == (3, 2, 8, 2)
    p = awq.linear_plan(16, 59392, 14848, 128)                  # and down: 58 groups, 464 bands
    assert (p["x_stage"], p["split_k"]) == (3, 8)
    assert awq.linear_workspace_bytes(16, 59392, 14848, 128) == 8 * 16 * 14848 * 4
    # one round of workgroups: two per CU with two tiles per wave, one with four
    assert awq.linear_plan(16, 32768, 16384, 128)["split_k"] == 8   # 64 groups x 8 = 512
    p = awq.linear_plan(32, 32768, 16384, 128)                      # above 16 rows: one tile, one per CU
    assert (p["tpw"], p["split_k"]) == (1, 2)                       # 128 groups x 2 = 256
    p = awq.linear_plan(16, 32768, 16384, 128, {"path": 1, "x_stage": 3, "tpw": 4})
    assert p["split_k"] == 8                                        # 32 groups x 8 = 256
    assert awq.linear_plan(16, 14848, 15872, 128)["x_stage"] == 2   # its QKV and O stay streamed
    assert awq.linear_plan(16, 14848, 14848, 128)["x_stage"] == 2
    assert awq.linear_plan(8, 14848, 59392, 128)["x_stage"] == 2    # fewer than 16 rows
    assert awq.linear_plan(32, 4096, 6144, 128)["x_stage"] == 2     # narrow
    assert awq.linear_plan(24, 4096, 28672, 64)["x_stage"] == 2     # G = 64
    p = awq.linear_silu_mul_plan(32, 4096, 28672, 128)         # gated: the same rule
    assert (p["x_stage"], p["tpw"], p["waves"], p["split_k"]) == (3, 2, 8, 2)
    assert awq.linear_silu_mul_plan(16, 4096, 28672, 128)["x_stage"] == 2
    p = awq.linear_plan(5, 384, 40, 128, {"path": 1, "x_stage": 3})
    assert (p["x_stage"], p["tpw"], p["waves"], p["split_k"]) == (3, 2, 8, 1)
    p = awq.linear_plan(5, 4096, 40, 128, {"path": 1, "x_stage": 3, "tpw": 4, "split_k": 5})
    assert (p["tpw"], p["split_k"]) == (4, 5)
    for bad in ({"path": 1, "x_stage": 3, "waves": 4},          # eight waves only
                {"path": 1, "x_stage": 3, "tpw": 3},            # one, two or four tiles per wave
                {"path": 1, "x_stage": 3, "tile": 2},
                {"path": 2, "x_stage": 3},                      # decode path only
                {"path": 1, "x_stage": 4}):
        with pytest.raises(awq.AWQError):
            awq.linear_plan(16, 4096, 4096, 128, bad)
    with pytest.raises(awq.AWQError):                           # at most 32 rows
        awq.linear_plan(33, 4096, 4096, 128, {"path": 1, "x_stage": 3})
    with pytest.raises(awq.AWQError):                           # whole groups per band
        awq.linear_plan(16, 4096, 4096, 64, {"path": 1, "x_stage": 3})
    with pytest.raises(awq.AWQError):                           # gated: two or four tiles per wave
        awq.linear_silu_mul_plan(16, 4096, 4096, 128, {"path": 1, "x_stage": 3, "tpw": 1})


def test_gated_plans(lib):
    import weight_only_bit_awq_amd as awq
    p = awq.linear_silu_mul_plan(1, 4096, 22016, 128)           # fused decode kernel, gate/up waves halved
    assert (p["path"], p["x_stage"], p["tpw"], p["waves"]) == (1, 1, 1, 8)
    assert awq.linear_silu_mul_plan(2048, 5120, 27648, 128)["path"] == 2
    # one or two rows: the staged fused kernel, with waves that let the
    # activations fit; more rows: the streamed one with gate and up tiles
    # paired; above 32 rows: the GEMM
    p = awq.linear_silu_mul_plan(2, 4096, 28672, 128)
    assert (p["path"], p["x_stage"], p["tpw"]) == (1, 1, 1)
    for M, tw in ((4, 4), (8, 4), (16, 4)):
        p = awq.linear_silu_mul_plan(M, 4096, 28672, 128)
        assert (p["path"], p["x_stage"], p["tpw"], p["waves"]) == (1, 2, tw, 4), (M, p)
    assert awq.linear_silu_mul_plan(32, 4096, 28672, 128)["x_stage"] == 3   # slab above 16 rows
    with pytest.raises(awq.AWQError):                            # two tile pairs need an even number per half
        awq.linear_silu_mul_plan(8, 1024, 96, 128, {"path": 1, "x_stage": 2, "tpw": 4})
    assert awq.linear_silu_mul_plan(40, 4096, 28672, 128)["path"] == 2
    assert awq.linear_silu_mul_workspace_bytes(2048, 5120, 27648, 128) == 0
    with pytest.raises(awq.AWQError):
        awq.linear_silu_mul_plan(1, 4096, 22000, 128)            # N % 32 != 0
    with pytest.raises(awq.AWQError):
        awq.linear_silu_mul_plan(1, 4096, 22016, 128, {"path": 1, "waves": 1})


def test_missing_library_raises(tmp_path, monkeypatch):
    import weight_only_bit_awq_amd as awq
    monkeypatch.setattr(awq, "_lib", None)
    monkeypatch.setattr(awq, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(awq.AWQLibraryMissing):
        awq.library()


def test_stream_read_validates_before_launch(lib):
    # nothing below reaches a kernel: empty, NULL, size and alignment errors
    assert lib.awq_stream_read(None, 0, None, None, None, None) == 0
    assert lib.awq_stream_read(None, 1024, ctypes.c_void_p(4096), None, None, None) == -1
    assert lib.awq_stream_read(ctypes.c_void_p(4096), 1000, ctypes.c_void_p(4096), None, None, None) == -2
    assert lib.awq_stream_read(ctypes.c_void_p(4104), 1024, ctypes.c_void_p(4096), None, None, None) == -4


def test_w4a8_validates_before_launch(lib):
    # an empty contraction (K = 0) writes y = 0: y is checked before that
    # fill is enqueued; empty outputs touch no pointer
    fake = ctypes.c_void_p(0x1000)
    assert lib.awq_linear_w4a8(None, None, None, None, 1, 0, 16, 128, None, None, 0, None) == -1
    assert lib.awq_linear_w4a8(None, None, None, None, 1, 0, 16, 128, ctypes.c_void_p(0x1008), None, 0, None) == -4
    assert lib.awq_linear_w4a8(None, None, None, None, 0, 0, 16, 128, None, None, 0, None) == 0
    assert lib.awq_linear_w4a8(fake, fake, fake, fake, 1, 128, 16, 128, None, None, 0, None) == -1
    assert lib.awq_linear_w4a8(fake, fake, fake, fake, 1, 100, 16, 128, fake, None, 0, None) == -2
    assert lib.awq_linear_w4a8(fake, fake, fake, fake, 1, 128, 16, 128, fake, None, 0, None) == -5


def _desc(**kw):
    import weight_only_bit_awq_amd as awq
    args = dict(B=1, q_heads=32, kv_heads=8, head_dim=128, capacity=4096, max_cached=4095)
    args.update(kw)
    return awq.attention_desc(args.pop("B"), args.pop("q_heads"), args.pop("kv_heads"), args.pop("head_dim"),
                              args.pop("capacity"), args.pop("max_cached"), **args)


def test_attention_validation_before_launch(lib):
    import weight_only_bit_awq_amd as awq
    sz = ctypes.c_size_t(0)

    def ws(**kw):
        return lib.awq_attention_workspace_bytes(ctypes.byref(_desc(**kw)), ctypes.byref(sz))

    assert ws() == 0 and sz.value > 0
    assert lib.awq_attention_workspace_bytes(None, ctypes.byref(sz)) == -1
    assert ws(head_dim=96) == -2                       # D must be 64 or 128
    assert ws(q_heads=30) == -2                        # Hq % Hkv
    assert ws(capacity=40, max_cached=10) == -2        # capacity % 32
    assert ws(max_cached=4096) == -2                   # max_cached < capacity
    assert ws(qkv_stride=100) == -2                    # stride below the row width
    assert ws(rope="half", theta=0.0) == -8            # theta > 0 with a rotation
    assert ws(rope="none", theta=0.0) == 0             # ... not needed without
    assert ws(scale=float("nan")) == -8
    assert ws(steps=-1) == -7
    d = _desc()
    d.rope_style = 3
    assert lib.awq_attention_workspace_bytes(ctypes.byref(d), ctypes.byref(sz)) == -8
    # the launch entry point: empty batch is a no-op; NULL, alignment and
    # workspace errors come back before anything is enqueued
    A = ctypes.c_void_p(4096)
    assert lib.awq_attention_decode(ctypes.byref(_desc(B=0)), None, None, None, None, None, None, 0, None) == 0
    assert lib.awq_attention_decode(ctypes.byref(_desc()), None, A, A, A, A, A, 1 << 30, None) == -1
    assert lib.awq_attention_decode(ctypes.byref(_desc()), ctypes.c_void_p(4104), A, A, A, A, A, 1 << 30,
                                    None) == -4
    need = awq.attention_workspace_bytes(_desc())
    assert lib.awq_attention_decode(ctypes.byref(_desc()), A, A, A, A, A, A, need - 1, None) == -5
    assert lib.awq_attention_decode(ctypes.byref(_desc()), A, A, A, A, A, ctypes.c_void_p(4096 + 16), need,
                                    None) == -4


@pytest.mark.parametrize("B,Hq,Hkv,D,S,maxc,steps", [
    (1, 32, 32, 128, 1024, 1023, 0), (1, 32, 8, 128, 4096, 4095, 0), (1, 71, 1, 64, 2048, 2047, 0),
    (16, 32, 32, 128, 2048, 2047, 0), (3, 12, 4, 64, 64, 0, 0), (2, 8, 2, 128, 512, 300, 3),
    (64, 32, 8, 128, 8192, 8000, 0)])
def test_attention_plans_cover_the_cache(lib, B, Hq, Hkv, D, S, maxc, steps):
    import weight_only_bit_awq_amd as awq
    d = _desc(B=B, q_heads=Hq, kv_heads=Hkv, head_dim=D, capacity=S, max_cached=maxc, steps=steps)
    pl = awq.attention_plan(d)
    if steps:
        assert pl["steps"] == steps
    # four waves per workgroup, 32 positions per step: every cached position
    # has a wave, and no workgroup starts past the bound
    covered = pl["workgroups_per_unit"] * 4 * pl["steps"] * 32
    assert covered >= max(maxc, 1) and covered - 4 * pl["steps"] * 32 < max(maxc, 1)
    T = -(-(Hq // Hkv) // 16)
    units = B * Hkv * T
    nbytes = awq.attention_workspace_bytes(d)
    # counters, then one state (16 heads x (D + 4) floats) per workgroup
    assert nbytes >= -(-units * 4 // 256) * 256 + units * pl["workgroups_per_unit"] * 16 * (D + 4) * 4
