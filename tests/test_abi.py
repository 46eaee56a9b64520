"""The C-ABI library on the host (no GPU needed): it loads, exports every
entry point the header declares, and rejects bad arguments with the right
status before touching a device."""

import ctypes
import os
import re

import pytest

import gqa_kv_cache_amd as G

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


def header_text():
    return re.sub(r"/\*.*?\*/", "", "\n".join(open(h).read() for h in HEADERS), flags=re.S)

# Fake, aligned device addresses: validation never dereferences pointers.
A16 = 0x10000


def declared_functions():
    return sorted(set(re.findall(r"\b(gqa_[a-z_]+)\s*\(", header_text())))


def test_library_exports_every_declared_function():
    lib = G.load_library()
    names = declared_functions()
    assert {"gqa_decode_run", "gqa_decode_workspace_size", "gqa_decode_make_plan", "gqa_resolve_rows",
            "gqa_status_string", "gqa_last_error", "gqa_abi_version", "gqa_kv_append",
            "gqa_kv_append_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_binding_argument_counts_match_header():
    text = header_text()
    lib = G.load_library()
    for name in declared_functions():
        m = re.search(r"\b" + name + r"\s*\((.*?)\)\s*;", text, flags=re.S)
        args = [a for a in m.group(1).split(",") if a.strip() and a.strip() != "void"]
        fn = getattr(lib, name)
        if fn.argtypes is not None:
            assert len(fn.argtypes) == len(args), f"{name}: binding has {len(fn.argtypes)} args, header {len(args)}"


def test_version_and_status_strings():
    assert G.gqa_abi_version() == 1
    for code, name in G.STATUS.items():
        assert G.gqa_status_string(code) == name


def base(**kw):
    d = dict(batch=2, s_q=1, h_q=8, h_kv=2, head_dim=128, max_seqlen_kv=100, seq_capacity=100,
             kv_rows=200, num_cus=256)
    d.update(kw)
    return G.make_params(**d)


BAD_SHAPES = [
    (dict(h_q=6, h_kv=4), 1),
    (dict(h_kv=0), 1),
    (dict(s_q=0), 2),
    (dict(s_q=65), 2),
    (dict(head_dim=96), 2),
    (dict(head_dim=512), 2),
    (dict(head_dim=256, math="valu"), 2),         # the VALU path is built for d <= 128
    (dict(h_q=1024, h_kv=1), 2),            # 1024 rows per KV head
    (dict(h_q=16, h_kv=1, s_q=64), 2),      # 1024 rows
    (dict(layout=7), 1),
    (dict(kv_dtype=3), 1),
    (dict(gate_mode=5), 1),
    (dict(max_seqlen_kv=-1), 1),
    (dict(seq_capacity=50), 1),             # capacity < max length
    (dict(kv_rows=100), 1),                 # batch * capacity > kv_rows
    (dict(kv_rows=0), 1),
    (dict(layout="paged", page_size=12, max_pages_per_seq=10, kv_rows=192), 2),
    (dict(layout="paged", page_size=16, max_pages_per_seq=2, kv_rows=192), 1),  # 32 < 100
    (dict(layout="paged", page_size=16, max_pages_per_seq=7, kv_rows=100), 1),  # not whole pages
    (dict(topk=-1), 1),
    (dict(kv_chunk=48), 1),
    (dict(kv_chunk=8192, layout="paged", page_size=16, max_pages_per_seq=7, kv_rows=224), 1),
    (dict(softmax_scale=float("inf")), 1),
    (dict(batch=70000), 1),
    (dict(math=3), 1),
    (dict(math="valu", h_q=16, h_kv=1), 2),         # 16 rows: more than the VALU path takes
    (dict(math="valu", h_q=8, h_kv=2, s_q=3), 2),   # 12 rows
]


@pytest.mark.parametrize("kw,status", BAD_SHAPES)
def test_plan_rejects_bad_shapes(kw, status):
    with pytest.raises(G.GqaError) as e:
        G.gqa_decode_make_plan(base(**kw))
    assert e.value.status == status, str(e.value)


def test_plan_never_sizes_an_expansion():
    # the workspace holds split partials only: O(splits * rows * d), never
    # O(S_kv * H_q * d) as a K/V expansion to the query-head count would
    p = base(batch=1, h_q=64, h_kv=8, s_q=2, max_seqlen_kv=131072, seq_capacity=131072, kv_rows=131072)
    plan = G.gqa_decode_make_plan(p)
    expansion = 2 * 131072 * 64 * 128 * 2
    assert plan["workspace_bytes"] < expansion / 100
    assert plan["workspace_bytes"] == G.gqa_decode_workspace_size(p)
    assert plan["rows"] == 16 and plan["row_blocks"] == 1 and plan["num_splits"] * plan["kv_chunk"] >= 131072


def test_plan_math_paths():
    # VALU computes 4 or 8 rows (at least the group's); MFMA 16-row blocks
    for rows_kw, rv in ((dict(h_q=8, h_kv=8), 1), (dict(h_q=8, h_kv=4), 2), (dict(h_q=8, h_kv=2), 4),
                        (dict(h_q=6, h_kv=2), 4), (dict(h_q=8, h_kv=1), 8), (dict(h_q=8, h_kv=4, s_q=3), 8)):
        plan = G.gqa_decode_make_plan(base(math="valu", **rows_kw))
        assert plan["math"] == 2 and plan["row_blocks"] == rv
    plan = G.gqa_decode_make_plan(base(math="mfma", h_q=8, h_kv=1))
    assert plan["math"] == 1 and plan["row_blocks"] == 1
    plan = G.gqa_decode_make_plan(base(math="auto", h_q=64, h_kv=2))   # 32 rows: MFMA only
    assert plan["math"] == 1 and plan["row_blocks"] == 2
    # the measured choice: MFMA at every row count (VALU only when asked for)
    assert G.gqa_decode_make_plan(base(math="auto", h_q=8, h_kv=8))["math"] == 1
    assert G.gqa_decode_make_plan(base(math="auto", h_q=8, h_kv=4))["math"] == 1


def test_plan_head_dim_256():
    # MFMA only; an auto plan with one row stays on MFMA for d = 256
    plan = G.gqa_decode_make_plan(base(head_dim=256, h_q=2, h_kv=2))
    assert plan["math"] == 1
    # paged d = 256: the auto chunk keeps the row table beside 128 KiB of tiles
    p = base(head_dim=256, h_q=32, h_kv=2, layout="paged", page_size=16, max_pages_per_seq=8192,
             max_seqlen_kv=131072, kv_rows=131072 * 2)
    plan = G.gqa_decode_make_plan(p)
    assert plan["kv_chunk"] <= 4032


def test_plan_heads_per_workgroup():
    # Paged and top-K lists with H_kv a multiple of 8 and one-byte K/V at d 128 (at most 16
    # rows): one workgroup covers all eight KV heads, so the grid holds one head group.
    kw = dict(batch=4, h_q=32, h_kv=8, kv_dtype="fp8_e4m3fn", max_seqlen_kv=512, seq_capacity=512, kv_rows=4 * 512)
    for extra in (dict(layout="paged", page_size=16, max_pages_per_seq=32), dict(topk=128)):
        plan = G.gqa_decode_make_plan(base(**kw, **extra))
        assert plan["partial_workgroups"] == plan["num_splits"] * 1 * 4, (extra, plan)
    # the same shape as a dense list, and bf16 d = 128 paged (two waves per SIMD do not
    # fit), keep four heads per workgroup: two head groups
    plan = G.gqa_decode_make_plan(base(**kw))
    assert plan["partial_workgroups"] == plan["num_splits"] * 2 * 4, plan
    plan = G.gqa_decode_make_plan(base(**dict(kw, kv_dtype="bf16"), layout="paged", page_size=16,
                                       max_pages_per_seq=32))
    assert plan["partial_workgroups"] == plan["num_splits"] * 2 * 4, plan
    # more than 16 rows: four heads
    plan = G.gqa_decode_make_plan(base(**dict(kw, h_q=256), layout="paged", page_size=16, max_pages_per_seq=32))
    assert plan["partial_workgroups"] % (plan["num_splits"] * 4) == 0 and plan["rows"] == 32


def test_plan_d256_two_row_blocks():
    # 32 rows at d 256: bf16 keeps Q in LDS with one KV head per workgroup (two head
    # groups for H_kv 2); FP8 has a head's two waves share the tiles, two heads per workgroup
    kw = dict(head_dim=256, h_q=32, h_kv=2, s_q=2, batch=1, max_seqlen_kv=131072, seq_capacity=131072,
              kv_rows=131072)
    plan = G.gqa_decode_make_plan(base(**kw, kv_dtype="bf16"))
    assert plan["row_blocks"] == 2 and plan["partial_workgroups"] == plan["num_splits"] * 2, plan
    plan = G.gqa_decode_make_plan(base(**kw, kv_dtype="fp8_e4m3fn"))
    assert plan["row_blocks"] == 2 and plan["partial_workgroups"] == plan["num_splits"] * 1, plan
    # a packed ragged bf16 cache keeps the shared tiles too
    plan = G.gqa_decode_make_plan(base(**dict(kw, seq_capacity=0), kv_dtype="bf16", layout="ragged"))
    assert plan["row_blocks"] == 2 and plan["partial_workgroups"] == plan["num_splits"], plan
    # paged bf16 with Q in LDS: the chunk leaves room for Q beside the tiles and the row table
    plan = G.gqa_decode_make_plan(base(**kw, kv_dtype="bf16", layout="paged", page_size=16, max_pages_per_seq=8192,
                                       topk=8192))
    assert plan["kv_chunk"] * 8 + 4096 + 16384 + 4 * 32768 + 512 <= 160 * 1024, plan


def test_plan_forced_chunk_and_single_split():
    p = base(kv_chunk=32)
    plan = G.gqa_decode_make_plan(p)
    assert plan["num_splits"] == 4 and plan["combine"] == 1 and plan["workspace_bytes"] > 0
    p = base(kv_chunk=128)
    plan = G.gqa_decode_make_plan(p)
    assert plan["num_splits"] == 1 and plan["combine"] == 0 and plan["workspace_bytes"] == 0


def _run(p, **ptrs):
    args = dict(q=A16, k=A16, v=A16, seqlens=A16, cu=None, bt=None, topk=None, ks=None, vs=None,
                gate=None, o=A16, lse=A16, ws=A16, ws_bytes=1 << 30)
    args.update(ptrs)
    lib = G.load_library()
    return lib.gqa_decode_run(ctypes.byref(p), args["q"], args["k"], args["v"], args["seqlens"], args["cu"],
                              args["bt"], args["topk"], args["ks"], args["vs"], args["gate"], args["o"],
                              args["lse"], args["ws"], ctypes.c_size_t(args["ws_bytes"]), None)


def test_run_validation_statuses():
    p = base()
    assert _run(p, q=None) == 1
    assert _run(p, seqlens=None) == 1
    assert _run(p, q=A16 + 2) == 3                       # misaligned
    assert _run(p, lse=A16 + 2) == 3
    assert _run(base(layout="ragged"), cu=None) == 1
    assert _run(base(layout="paged", page_size=16, max_pages_per_seq=7, kv_rows=224)) == 1  # no block table
    assert _run(base(topk=8)) == 1                        # no topk_idx
    assert _run(base(kv_dtype="fp8_e4m3fn")) == 1          # no scales
    assert _run(base(gate_mode="elementwise")) == 1        # no gate
    assert _run(base(gate_mode="elementwise"), gate=A16 + 4) == 3
    assert _run(base(kv_chunk=32), ws=None) == 4           # workspace needed
    assert _run(base(kv_chunk=32), ws_bytes=16) == 4
    msg = G.load_library().gqa_last_error().decode()
    assert "workspace" in msg


def test_run_batch_zero_is_a_no_op():
    assert _run(base(batch=0, kv_rows=1)) == 0


# ---- K/V append -----------------------------------------------------------

def append_base(**kw):
    d = dict(batch=2, s_new=3, h_kv=4, head_dim=128, layout="paged", kv_dtype="fp8_e4m3fn",
             scale_policy="given", kv_rows=4096, page_size=16, max_pages_per_seq=8)
    d.update(kw)
    return G.make_append_params(**d)


def _append(p, kn=A16, vn=A16, sl=A16, so=None, bt=A16, kc=A16, vc=A16, ks=A16, vs=A16, ws=None, ws_bytes=0):
    lib = G.load_library()
    return lib.gqa_kv_append(ctypes.byref(p), kn, vn, sl, so, bt, kc, vc, ks, vs, ws, ctypes.c_size_t(ws_bytes), None)


def test_append_params_layout_matches_header():
    assert ctypes.sizeof(G.AppendParams) == 64


@pytest.mark.parametrize("kw,status", [
    (dict(s_new=0), 1), (dict(batch=-1), 1), (dict(h_kv=0), 2), (dict(h_kv=257), 2), (dict(head_dim=96), 2),
    (dict(kv_dtype=7), 1), (dict(scale_policy=3), 1), (dict(kv_rows=0), 1), (dict(layout="ragged"), 2),
    (dict(page_size=12), 1), (dict(max_pages_per_seq=0), 1), (dict(layout="contiguous", seq_capacity=0), 1),
    (dict(layout="contiguous", seq_capacity=4096), 1),   # batch * capacity > kv_rows
])
def test_append_rejects_bad_params(kw, status):
    n = ctypes.c_size_t(0)
    assert G.load_library().gqa_kv_append_workspace_size(ctypes.byref(append_base(**kw)), ctypes.byref(n)) == status
    assert _append(append_base(**kw)) == status


def test_append_reserved_must_be_zero():
    p = append_base()
    p.reserved[2] = 1
    assert _append(p) == 1


def test_append_validation_statuses():
    p = append_base()
    assert _append(p, kn=None) == 1
    assert _append(p, sl=None) == 1
    assert _append(p, bt=None) == 1                              # paged needs a block table
    assert _append(p, ks=None) == 1                              # FP8 needs scales
    assert _append(p, so=A16) == 1                               # seqlens_out aliases seqlens
    assert _append(p, kc=A16 + 8) == 3
    assert _append(p, so=A16 + 2) == 3


def test_append_workspace_only_for_multi_block_first_block():
    ws = G.gqa_kv_append_workspace_size
    assert ws(append_base(scale_policy="first_block")) == 0                 # one workgroup per request
    assert ws(append_base(scale_policy="given", s_new=5000)) == 0
    assert ws(append_base(kv_dtype="bf16", scale_policy="first_block", s_new=5000)) == 0
    need = ws(append_base(scale_policy="first_block", s_new=5000))
    assert need == 2 * 40 * 2 * 4 * 4           # B x chunks (5000 rows / 128 per workgroup) x (K, V) x H_kv x 4 B
    assert _append(append_base(scale_policy="first_block", s_new=5000)) == 4
    assert _append(append_base(scale_policy="first_block", s_new=5000), ws=A16, ws_bytes=need - 4) == 4


def test_append_batch_zero_is_a_no_op():
    assert _append(append_base(batch=0)) == 0


def test_plan_tiling_of_large_groups():
    # rows -> 16-row blocks per KV head: four waves of one block up to 64
    # rows; beyond, eight waves of one block (128 rows per row group) or of
    # two (d <= 128, more than 128 rows: 256 per row group); bf16 at d = 64
    # keeps four waves (row groups of 64) up to 256 rows
    def plan(**kw):
        d = dict(batch=1, s_q=1, h_q=8, h_kv=8, head_dim=128, max_seqlen_kv=4096, seq_capacity=4096,
                 kv_rows=4096, num_cus=256)
        d.update(kw)
        return G.gqa_decode_make_plan(G.make_params(**d))
    assert plan(h_q=48, h_kv=1)["row_blocks"] == 4                       # 48 rows: 4 waves x 1 block
    assert plan(h_q=64, h_kv=8, s_q=16)["row_blocks"] == 8               # 128 rows: 8 waves x 1
    assert plan(h_q=96, h_kv=1)["row_blocks"] == 8                       # 96 rows: 8 x 1, 2 blocks idle
    assert plan(h_q=64, h_kv=8, s_q=64)["row_blocks"] == 32              # 512 rows: 2 row groups of 8 x 2
    assert plan(h_q=64, h_kv=8, s_q=64, head_dim=256)["row_blocks"] == 32  # d256: 4 row groups of 8 x 1
    assert plan(h_q=32, h_kv=2, s_q=2, head_dim=256)["row_blocks"] == 2  # two waves x 1 block
    assert plan(h_q=32, h_kv=2, s_q=2, head_dim=256, kv_dtype="fp8_e4m3fn")["row_blocks"] == 2
    assert plan(h_q=64, h_kv=8, s_q=16, head_dim=64)["row_blocks"] == 8  # bf16 d64, 128 rows: 2 x (4 x 1)
    assert plan(h_q=80, h_kv=1, s_q=2, head_dim=64)["row_blocks"] == 12  # bf16 d64, 160 rows: 3 x (4 x 1)
    assert plan(h_q=64, h_kv=1, s_q=8, head_dim=64)["row_blocks"] == 32  # bf16 d64, 512 rows: 2 x (8 x 2)
    fp8_d64 = dict(head_dim=64, kv_dtype="fp8_e4m3fn")
    assert plan(h_q=80, h_kv=1, **fp8_d64)["row_blocks"] == 8            # 80 rows, odd H_kv: 8 x 1
    assert plan(h_q=48, h_kv=1, **fp8_d64)["row_blocks"] == 4            # 48 rows, odd H_kv: 1 wave x 4
    assert plan(h_q=96, h_kv=2, **fp8_d64)["row_blocks"] == 4            # 48 rows, even H_kv: 2 waves x 2
    p1, p4 = plan(h_q=64, h_kv=8, s_q=2), plan(h_q=64, h_kv=8, s_q=64)
    assert p4["partial_workgroups"] >= p1["partial_workgroups"]
