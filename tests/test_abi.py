"""C ABI checks that need no GPU: the library loads, exports every entry
point include/densegemm.h declares, the Python struct mirrors the C layout,
and every invalid descriptor is rejected on the host before any launch."""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import dense_gemm_10_amd as dg
import workloads as W
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "densegemm.h")

# Fake, never-dereferenced device addresses: every call below returns during
# host validation, before anything is enqueued.
PA, PB, PC, PW = 0x100000, 0x200000, 0x300000, 0x400000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    names = _declared_functions()
    assert set(names) >= {"dg_gemm", "dg_gemm_workspace_size", "dg_gemm_describe",
                          "dg_status_string", "dg_version", "dg_schedule_map"}
    lib = ctypes.CDLL(dg.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", dg.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dg_\w+)", out))
    assert exported == set(names)


def test_struct_layout_matches_header():
    fields = [f for f, _ in dg.DgGemmDesc._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"',
           'int main(void) {', 'printf("%zu\\n", sizeof(dg_gemm_desc));']
    for f in fields:
        src.append(f'printf("%zu\\n", offsetof(dg_gemm_desc, {f}));')
    src.append("return 0; }")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(src))
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", c, "-o", exe], check=True)
        vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True,
                                               check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(dg.DgGemmDesc)
    for f, off in zip(fields, vals[1:]):
        assert getattr(dg.DgGemmDesc, f).offset == off, f


def test_version_and_status_strings():
    assert dg.dg_version() == 10000
    for code, name in [(0, "DG_SUCCESS"), (1, "DG_ERROR_INVALID_VALUE"),
                       (2, "DG_ERROR_NOT_SUPPORTED"), (3, "DG_ERROR_INSUFFICIENT_WORKSPACE"),
                       (4, "DG_ERROR_LAUNCH")]:
        assert dg.dg_status_string(code) == name
    assert dg.dg_status_string(99) == "DG_ERROR_UNKNOWN"


def _desc(**kw):
    base = dict(M=64, N=48, K=32, a_type="f32")
    base.update(kw)
    return dg.make_desc(**base)


def _gemm_status(d, A=PA, B=PB, C=PC, ws=None, ws_bytes=0):
    return dg.dg_gemm(d, A, B, C, ws, ws_bytes, None, check=False)


INVALID = [
    ("negative M", dict(M=-1)),
    ("negative K", dict(K=-3)),
    ("negative batch", dict(batch=-1)),
    ("bad a_type", dict(a_type=7)),
    ("bad order", dict(a_order=2)),
    ("bad act", dict(act=9)),
    ("bad algo", dict(algo=11)),
    ("negative split", dict(split_k=-1)),
    ("negative group", dict(group_m=-2)),
    ("bad xcd flag", dict(xcd_remap=3)),
    ("lda below K (row-major A)", dict(lda=31)),
    ("lda below M (col-major A)", dict(a_order="col", lda=63)),
    ("ldb below N (row-major B)", dict(ldb=47)),
    ("ldb below K (col-major B)", dict(b_order="col", ldb=31)),
    ("ldc below N", dict(ldc=47)),
    ("ldc below M (col-major C)", dict(c_order="col", ldc=63)),
    ("zero ld", dict(lda=0)),
    ("negative stride", dict(stride_a=-8)),
    ("C batches overlap", dict(batch=2, stride_c=100)),
    ("C broadcast", dict(batch=2, stride_c=0)),
    ("size overflow", dict(M=2 ** 40, N=2 ** 40, K=1, lda=1, ldb=2 ** 40, ldc=2 ** 40)),
]


@pytest.mark.parametrize("what,kw", INVALID, ids=[w for w, _ in INVALID])
def test_invalid_descriptors_rejected_before_launch(what, kw):
    d = _desc(**kw)
    assert _gemm_status(d) == dg.DG_ERROR_INVALID_VALUE
    with pytest.raises(dg.DgError) as e:
        dg.dg_gemm_workspace_size(d)
    assert e.value.status == dg.DG_ERROR_INVALID_VALUE


def test_bad_struct_size():
    d = _desc()
    d.struct_size = 12
    assert _gemm_status(d) == dg.DG_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [dict(a_type="f32", b_type="bf16"),
                                dict(a_type="bf16", b_type="f32"),
                                dict(a_type="f32", c_type="bf16"),
                                dict(a_type="f16", b_type="bf16"),
                                dict(a_type="f32", c_type="f16"),
                                dict(split_k=100000)])
def test_unsupported_combinations(kw):
    assert _gemm_status(_desc(**kw)) == dg.DG_ERROR_NOT_SUPPORTED


def test_pointer_rules():
    d = _desc()
    assert _gemm_status(d, C=None) == dg.DG_ERROR_INVALID_VALUE
    assert _gemm_status(d, A=None) == dg.DG_ERROR_INVALID_VALUE
    assert _gemm_status(d, B=None) == dg.DG_ERROR_INVALID_VALUE
    assert _gemm_status(d, A=PA + 2) == dg.DG_ERROR_INVALID_VALUE    # fp32 needs 4-byte alignment
    bd = _desc(a_type="bf16")
    assert _gemm_status(bd, C=PC + 1) == dg.DG_ERROR_INVALID_VALUE
    # C overlapping A or B
    assert _gemm_status(d, C=PA + 4) == dg.DG_ERROR_INVALID_VALUE
    assert _gemm_status(d, C=PB - 16) == dg.DG_ERROR_INVALID_VALUE
    # C overlapping the bias vector
    dbias = _desc(bias=PC + 8)
    assert _gemm_status(dbias) == dg.DG_ERROR_INVALID_VALUE


def test_noop_shapes_succeed_without_launch():
    for kw in [dict(M=0), dict(N=0), dict(batch=0)]:
        d = _desc(**kw)
        assert _gemm_status(d, A=None, B=None, C=None) == dg.DG_SUCCESS
        assert dg.dg_gemm_workspace_size(d) == 0
        assert dg.dg_gemm_describe(d) == "noop"


def test_forced_split_needs_workspace():
    d = _desc(K=4096, split_k=4)
    need = dg.dg_gemm_workspace_size(d)
    assert need == 4 * 64 * 48 * 4
    # 64 * 48 outputs, N a multiple of 4: four per thread, 1024 per block
    assert "reduce_blocks=3 " in dg.dg_gemm_describe(d, need)
    d47 = _desc(K=4096, N=47, ldb=47, ldc=47, split_k=4)            # one output per thread
    assert "reduce_blocks=12 " in dg.dg_gemm_describe(d47, dg.dg_gemm_workspace_size(d47))
    assert _gemm_status(d) == dg.DG_ERROR_INSUFFICIENT_WORKSPACE
    assert _gemm_status(d, ws=PW, ws_bytes=need - 4) == dg.DG_ERROR_INSUFFICIENT_WORKSPACE
    # workspace overlapping C
    assert _gemm_status(d, ws=PC, ws_bytes=need) == dg.DG_ERROR_INVALID_VALUE


def test_noalloc_refuses_forced_plans_beyond_its_scratch():
    """dg_gemm_noalloc plans against DG_NOALLOC_SCRATCH_BYTES and refuses a
    forced split-K whose workspace exceeds it, on the host, before any
    runtime call (fake, far-apart addresses: nothing is dereferenced)."""
    A, B, C = 1 << 40, 2 << 40, 3 << 40
    d = _desc(M=4096, N=4096, K=4096, lda=4096, ldb=4096, ldc=4096, split_k=2)
    assert dg.dg_gemm_workspace_size(d) > dg.DG_NOALLOC_SCRATCH_BYTES
    assert dg.dg_gemm_noalloc(d, A, B, C, check=False) == dg.DG_ERROR_INSUFFICIENT_WORKSPACE
    # validation errors come first, as for dg_gemm
    assert dg.dg_gemm_noalloc(d, A, B, None, check=False) == dg.DG_ERROR_INVALID_VALUE
    bad = _desc(M=-1)
    assert dg.dg_gemm_noalloc(bad, A, B, C, check=False) == dg.DG_ERROR_INVALID_VALUE
    assert dg.dg_gemm_noalloc(_desc(M=0), None, None, None, check=False) == dg.DG_SUCCESS


def _desc_for(p, **kw):
    f = W.desc_fields(p)
    f.update(kw)
    return dg.make_desc(**f)


def test_plans_of_the_five_workloads(monkeypatch):
    # the heuristic plans (the offline-tuned table switched off)
    monkeypatch.setenv("DG_TUNED", "0")
    c1 = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["c1"]))
    assert "kernel=mfma_f32" in c1 and "splits=1" in c1 and "bm=128" in c1
    c2 = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["c2"]))
    assert "kernel=mfma_f32" in c2 and "programs=256" in c2
    c2v = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["c2"], algo=dg.DG_ALGO_VALU_F32))
    # 512 blocks of 128 x 256 fill the two resident blocks per CU exactly
    assert "kernel=valu_f32" in c2v and "tile=valu_f32_128x256x16_t8x16" in c2v and "programs=512" in c2v
    c1v = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["c1"], algo=dg.DG_ALGO_VALU_F32))
    assert "tile=valu_f32_128x128x16_t8x8" in c1v
    c3 = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["c3"]))
    assert "kernel=mfma_bf16" in c3 and "bm=256 bn=256" in c3 and "programs=256" in c3
    c4 = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["c4"]))
    # 272 tiles of 256^2 quantise badly, so the full plan takes 128^2 tiles;
    # N = 4097 leaves one column past the last full one: the full columns
    # (32 x 32 tiles of 128^2, two waves) run tiled, the last one as a sliver
    assert "kernel=mfma_bf16" in c4 and "bm=128 bn=128" in c4 and "programs=1024" in c4
    assert "sliver=1" in c4 and "schedule=data_parallel" in c4
    d5 = _desc_for(W.WORKLOADS["c5"])
    ws = dg.dg_gemm_workspace_size(d5)
    assert ws > 0
    c5 = dg.dg_gemm_describe(d5, ws)
    assert "kernel=mfma_bf16" in c5 and "splits=1 " not in c5
    # without workspace the automatic choice does not split
    assert "splits=1 " in dg.dg_gemm_describe(d5, 0)
    # the tuned plan of the ragged GELU GEMM: a stream-K entry keeps the
    # whole grid (its tail wave sliced) when workspace is given; without
    # workspace, or with a data-parallel entry, the entry plans the full
    # columns and the last column is a sliver
    monkeypatch.delenv("DG_TUNED")
    p4 = W.WORKLOADS["c4"]
    entry = [e for e in _tuned_entries() if e[:5] == ("KERNEL_MFMA_BF16", p4.M, p4.N, p4.K, 1)]
    assert len(entry) == 1
    d4 = _desc_for(p4)
    t4 = dg.dg_gemm_describe(d4, dg.dg_gemm_workspace_size(d4))
    assert "tuned=1" in t4 and f"tile={entry[0][5]} " in t4
    if entry[0][6] == "DG_SCHED_STREAM_K":
        assert "schedule=stream_k" in t4 and "sliver=0" in t4
    else:
        assert "schedule=data_parallel" in t4 and "sliver=1" in t4
    t4 = dg.dg_gemm_describe(d4, 0)
    assert "tuned=1" in t4 and f"tile={entry[0][5]} " in t4
    assert "schedule=data_parallel" in t4 and "sliver=1" in t4


def test_f16_plans(monkeypatch):
    f = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["f16_4096"]))
    assert "kernel=mfma_f16" in f and "tile=mfma_f16_256x256x64_w2x2_s2" in f
    g = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["f16_gelu"]))
    # the fp16 family has the bf16 family's tiles, and the tuned table uses them
    assert "kernel=mfma_f16" in g and "tuned=1" in g and "tile=mfma_f16_" in g
    monkeypatch.setenv("DG_TUNED", "0")
    g0 = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["f16_gelu"]))
    assert "kernel=mfma_f16" in g0 and "tile=mfma_f16_128x128x32_w2x2_s4" in g0
    monkeypatch.delenv("DG_TUNED")
    # every output type is accepted for 16-bit inputs
    for a in ("bf16", "f16"):
        for c in ("f32", "bf16", "f16"):
            d = _desc(a_type=a, b_type=a, c_type=c, b_order="col", bias=PW, bias_type="f16")
            assert f"kernel=mfma_{a}" in dg.dg_gemm_describe(d)
    # each 16-bit family takes only its own element type
    for a, algo in (("f16", dg.DG_ALGO_MFMA_BF16), ("bf16", dg.DG_ALGO_MFMA_F16),
                    ("f32", dg.DG_ALGO_MFMA_F16)):
        with pytest.raises(dg.DgError) as e:
            dg.dg_gemm_describe(_desc(a_type=a, b_type=a, b_order="col", algo=algo))
        assert e.value.status == dg.DG_ERROR_NOT_SUPPORTED
    # fp16 in any order of A and B goes to its matrix-core kernel; with a
    # leading dimension off the 16-byte grid, to the generic kernel
    assert "kernel=mfma_f16" in dg.dg_gemm_describe(_desc(a_type="f16", b_type="f16"))
    assert "kernel=generic" in dg.dg_gemm_describe(_desc(a_type="f16", b_type="f16", lda=36))
    # fp16 pointers need 2-byte alignment
    assert _gemm_status(_desc(a_type="f16", b_type="f16", c_type="f16"), C=PC + 1) == \
        dg.DG_ERROR_INVALID_VALUE
    # forced stream-K on the fp16 kernel
    # (N = 4352: 16 x 17 tiles of 256^2, no sliver columns, a thin last wave)
    sk = dg.dg_gemm_describe(_desc_for(W.WORKLOADS["f16_gelu"].replace(K=4096, N=4352)),
                             1 << 34)
    assert "kernel=mfma_f16" in sk and "schedule=stream_k" in sk and "bm=256" in sk


def test_layouts_outside_the_fast_paths_use_the_generic_kernel():
    assert "kernel=generic" in dg.dg_gemm_describe(_desc(lda=33))     # ld not a multiple of 4
    d = _desc(a_type="bf16", b_order="col", lda=36)                    # lda not a multiple of 8
    assert "kernel=generic" in dg.dg_gemm_describe(d)
    for bad in [_desc(a_type="bf16", lda=36, algo=dg.DG_ALGO_MFMA_BF16),  # lda % 8 != 0
                _desc(lda=33, algo=dg.DG_ALGO_MFMA_F32),                  # ld not a multiple of 4
                _desc(lda=33, algo=dg.DG_ALGO_VALU_F32),
                _desc(a_type="bf16", b_order="col", algo=dg.DG_ALGO_VALU_F32)]:
        with pytest.raises(dg.DgError) as e:
            dg.dg_gemm_describe(bad)
        assert e.value.status == dg.DG_ERROR_NOT_SUPPORTED


@pytest.mark.parametrize("a_order,b_order", [("row", "row"), ("col", "col"), ("col", "row"),
                                             ("row", "col")])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_every_16bit_layout_runs_on_the_matrix_cores(a_order, b_order, dt, monkeypatch):
    """Any order of A and B takes the 16-bit matrix-core kernel; an M- or
    N-contiguous operand only on the two tiles of the automatic choice,
    whatever the tuned table or a forced tile say."""
    fam = "mfma_bf16" if dt == "bf16" else "mfma_f16"
    for M, N, K, tile in [(4096, 4096, 4096, "256x256"), (300, 260, 200, "128x128")]:
        up8 = lambda v: -(-v // 8) * 8     # noqa: E731
        d = dg.make_desc(M, N, K, a_type=dt, a_order=a_order, b_order=b_order, c_type=dt,
                         lda=up8(K if a_order == "row" else M),
                         ldb=up8(N if b_order == "row" else K))
        text = dg.dg_gemm_describe(d, 1 << 34)
        assert f"kernel={fam}" in text and f"tile={fam}_{tile}" in text, text
    if (a_order, b_order) != ("row", "col"):
        monkeypatch.setenv("DG_FORCE_TILE", f"{fam}_256x128x32_w2x2_s4")
        d = dg.make_desc(4096, 4096, 4096, a_type=dt, a_order=a_order, b_order=b_order)
        text = dg.dg_gemm_describe(d, 1 << 34)
        assert "tile=" + fam + "_256x256" in text or "tile=" + fam + "_128x128" in text, text
        assert "tuned=0" in text


def test_batch_strides_ignored_for_a_single_matrix():
    # odd strides do not matter when batch == 1 ...
    d = _desc(M=64, N=48, K=32, stride_a=12345, stride_b=777)
    assert "kernel=mfma_f32" in dg.dg_gemm_describe(d)
    # ... but do when there is a batch
    d = _desc(M=64, N=48, K=32, batch=2, stride_a=12345, stride_b=777 * 4)
    assert "kernel=generic" in dg.dg_gemm_describe(d)


def test_k_zero_and_alpha_zero_never_split():
    assert "splits=1 " in dg.dg_gemm_describe(_desc(K=0, split_k=8, lda=1), 1 << 30)
    assert "splits=1 " in dg.dg_gemm_describe(_desc(K=8192, alpha=0.0, split_k=8), 1 << 30)


def _sk_fields(text):
    kv = dict(t.split("=", 1) for t in text.split() if "=" in t)
    return {k: int(kv[k]) for k in ("dp_tiles", "tail_tiles", "tail_splits", "tail_k_per_split")}


def test_stream_k_plan_for_a_badly_quantised_grid(monkeypatch):
    # the heuristic (tuned table off) on a grid like the GELU workload's
    # with a long K (the automatic choice wants K >= 2048) and N = 4352, so
    # that no sliver columns are split off
    monkeypatch.setenv("DG_TUNED", "0")
    d = _desc_for(W.WORKLOADS["c4"].replace(K=4096, N=4352))
    ws = dg.dg_gemm_workspace_size(d)
    text = dg.dg_gemm_describe(d, ws)
    # with stream-K taking the tail wave the large tile is kept: 4095 x 4352
    # in 256 x 256 tiles = 16 x 17 = 272 = one wave of 256 + 16 tail tiles
    assert "schedule=stream_k" in text and "bm=256 bn=256" in text
    sk = _sk_fields(text)
    assert sk["dp_tiles"] == 256 and sk["tail_tiles"] == 16
    assert sk["tail_splits"] == 16 and sk["tail_k_per_split"] == 256   # K = 4096
    assert "programs=%d " % (256 + 16 * 16) in text
    assert "fixup_blocks=%d " % (16 * 64) in text
    assert ws == 16 * 16 * 256 * 256 * 4
    # without workspace, or with K < 2048, the automatic choice stays data-parallel
    assert "schedule=data_parallel" in dg.dg_gemm_describe(d, 0)
    assert "schedule=data_parallel" in dg.dg_gemm_describe(_desc_for(W.WORKLOADS["c4"]), 1 << 34)
    # a whole number of waves stays data-parallel
    assert "schedule=data_parallel" in dg.dg_gemm_describe(_desc_for(W.WORKLOADS["c3"]), 1 << 30)


def test_stream_k_slices_cover_k_once():
    for M, N, K in [(4095, 4097, 1000), (640, 640, 1024), (2944, 2944, 4096), (4352, 4352, 200)]:
        d = _desc(M=M, N=N, K=K, a_type="bf16", b_order="col", schedule=dg.DG_SCHED_STREAM_K)
        sk = _sk_fields(dg.dg_gemm_describe(d, 1 << 34))
        S, kps = sk["tail_splits"], sk["tail_k_per_split"]
        assert S >= 2 and kps % 32 == 0
        assert (S - 1) * kps < K <= S * kps          # every slice non-empty, all of K covered


def test_stream_k_requirements():
    sk = dict(schedule=dg.DG_SCHED_STREAM_K)
    # only the 16-bit matrix-core kernels, one matrix
    for bad in [_desc(**sk), _desc(a_type="bf16", b_order="col", batch=2, **sk)]:
        with pytest.raises(dg.DgError) as e:
            dg.dg_gemm_describe(bad, 1 << 30)
        assert e.value.status == dg.DG_ERROR_NOT_SUPPORTED
    # under stream-K, split_k sets the K slices of each tail tile (one K step
    # at least each): 3000 x 3000 in 256 x 256 tiles is 144 tiles, all in the
    # tail
    for S, want in [(4, 4), (8, 8), (100, 64)]:              # K = 4096 is 64 K steps of 64
        t = dg.dg_gemm_describe(_desc(M=3000, N=3000, K=4096, a_type="bf16", b_order="col",
                                      split_k=S, **sk), 1 << 34)
        kv = _sk_fields(t)
        assert "splits=1 " in t and "bm=256" in t, t
        assert kv["tail_splits"] == want and kv["tail_tiles"] == 144, t
    d = _desc(M=3000, N=3000, K=256, a_type="bf16", b_order="col", **sk)
    need = dg.dg_gemm_workspace_size(d)
    assert need > 0
    big = dict(A=1 << 40, B=2 << 40, C=3 << 40)     # far apart: no operand overlap
    assert _gemm_status(d, **big) == dg.DG_ERROR_INSUFFICIENT_WORKSPACE
    assert _gemm_status(d, ws=4 << 40, ws_bytes=need - 16, **big) == \
        dg.DG_ERROR_INSUFFICIENT_WORKSPACE
    assert _gemm_status(d, ws=(4 << 40) + 8, ws_bytes=need, **big) == \
        dg.DG_ERROR_INVALID_VALUE                    # the workspace must be 16-byte aligned
    bad = _desc(schedule=3)
    assert _gemm_status(bad) == dg.DG_ERROR_INVALID_VALUE
    # data-parallel on request
    d4 = _desc_for(W.WORKLOADS["c4"], schedule=dg.DG_SCHED_DATA_PARALLEL)
    assert "schedule=data_parallel" in dg.dg_gemm_describe(d4, 1 << 34)


def _tuned_entries():
    import re
    path = os.path.join(ROOT, "dense_gemm_10_amd", "csrc", "tuned_table.inc")
    text = open(path).read()
    pat = (r'\{(KERNEL_\w+), (\d+), (\d+), (\d+), (\d+), "([\w]+)", (DG_SCHED_\w+), '
           r'(\d+)\},')
    return [(k, int(M), int(N), int(K), int(b), t, s, int(S)) for k, M, N, K, b, t, s, S in
            re.findall(pat, text)]


def test_tuned_table_entries_are_what_the_planner_picks(monkeypatch):
    import itertools
    from dense_gemm_10_amd.tune import shapes
    by_shape = {(p.M, p.N, p.K, p.batch, p.a_type): p for p in shapes()}
    fam_type = {"KERNEL_MFMA_BF16": "bf16", "KERNEL_MFMA_F16": "f16", "KERNEL_MFMA_F32": "f32"}
    entries = _tuned_entries()
    for kern, M, N, K, b, tile, sched, splits in entries:
        p = by_shape[(M, N, K, b, fam_type[kern])]        # every entry comes from a swept shape
        d = _desc_for(p)
        ws = dg.dg_gemm_workspace_size(d)
        text = dg.dg_gemm_describe(d, ws)
        assert "tuned=1" in text and f"tile={tile} " in text, (p.name, text)
        if sched == "DG_SCHED_DATA_PARALLEL":
            assert "schedule=data_parallel" in text, (p.name, text)
            if splits:
                assert f" splits={splits} " in text, (p.name, text)
        else:
            assert "schedule=stream_k" in text, (p.name, text)
            if splits:
                assert f"tail_splits={splits} " in text, (p.name, text)
        # DG_TUNED=0 gives the heuristic plan, DG_FORCE_TILE overrides the table
        monkeypatch.setenv("DG_TUNED", "0")
        assert "tuned=0" in dg.dg_gemm_describe(d, ws)
        monkeypatch.delenv("DG_TUNED")
    # a shape next to a tuned one is not matched
    for kern, M, N, K, b, tile, sched, splits in itertools.islice(entries, 3):
        p = by_shape[(M, N, K, b, fam_type[kern])].replace(K=K + 8)
        assert "tuned=0" in dg.dg_gemm_describe(_desc_for(p), 1 << 34)
