"""C-ABI checks that need no GPU: the library loads and exports every symbol the
header declares, the ctypes structs match the C layout, and every host-checkable
argument error returns its own status before anything is enqueued (the fake
device addresses below are never dereferenced: checks fail first).
"""
import ctypes
import os
import re
import subprocess
from ctypes import POINTER, c_int32, c_void_p

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qd.h")

Q = pytest.importorskip("decode_step_amd.qd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(Q.LIB_PATH):
        from decode_step_amd import build as B
        B.build()
    return Q.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qd_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["qd_decode_step", "qd_prefill_block", "qd_kv_append", "qd_workspace_bytes", "qd_quantize_rows_int8",
              "qd_last_error", "qd_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", Q.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(qd_\w+)", out))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)
    assert lib.qd_abi_version() == Q.ABI_VERSION == 5


def test_struct_layout_matches_the_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "qd.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(qd_config),'
                   ' sizeof(qd_layer), sizeof(qd_weights), sizeof(qd_kv),'
                   ' offsetof(qd_kv, max_blocks), offsetof(qd_config, rms_eps)); return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    want = [ctypes.sizeof(Q.qd_config), ctypes.sizeof(Q.qd_layer), ctypes.sizeof(Q.qd_weights),
            ctypes.sizeof(Q.qd_kv), Q.qd_kv.max_blocks.offset, Q.qd_config.rms_eps.offset]
    assert got == want


# ---------------------------------------------------------------- host-side errors

FAKE = 0x7f0000000000   # 16-byte aligned, never dereferenced


def _cfg(**over):
    d = dict(n_layers=1, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=96, vocab=100,
             page_size=16, rms_eps=1e-6, rope_theta=1e6, qk_norm=0, w_dtype=Q.QD_BF16,
             kv_dtype=Q.QD_BF16)
    d.update(over)
    return Q.qd_config(**d)


class Fixture:
    def __init__(self, cfg, pos=(5,), table=None, num_pages=4, max_blocks=2):
        self.cfg = cfg
        L = cfg.n_layers
        self.layers = (Q.qd_layer * L)()
        for l in range(L):
            for i, n in enumerate(Q.LAYER_FIELDS):
                if n not in ("bq", "bk", "bv", "q_norm", "k_norm"):
                    setattr(self.layers[l], n, FAKE + 4096 * i)
        self.w = Q.qd_weights(FAKE, FAKE, FAKE, ctypes.cast(self.layers, POINTER(Q.qd_layer)))
        self.kp = (c_void_p * L)(*([FAKE] * L))
        self.vp = (c_void_p * L)(*([FAKE] * L))
        B = len(pos)
        t = np.zeros((B, max_blocks), np.int32) if table is None else np.asarray(table, np.int32)
        self.table = np.ascontiguousarray(t)
        self.kv = Q.qd_kv(ctypes.cast(self.kp, POINTER(c_void_p)), ctypes.cast(self.vp, POINTER(c_void_p)),
                          FAKE, self.table.ctypes.data_as(POINTER(c_int32)), max_blocks, num_pages)
        self.pos = np.ascontiguousarray(pos, np.int32)

    def decode(self, batch=None, tokens=FAKE, x_in=None, ws=FAKE, ws_bytes=1 << 40, logits=FAKE,
               pos_host=True, pos=FAKE, next_tokens=None, x_out=None, layer_out=None):
        B = len(self.pos) if batch is None else batch
        ph = self.pos.ctypes.data_as(POINTER(c_int32)) if pos_host else None
        return Q.qd_decode_step(self.cfg, self.w, self.kv, B, tokens, x_in, pos, ph, logits, next_tokens,
                                x_out, layer_out, ws, ws_bytes, None)


def _expect(status, what):
    assert status == what, (Q.STATUS_NAMES.get(status), Q.qd_last_error())
    assert Q.qd_last_error() != ""


def test_null_config(lib):
    f = Fixture(_cfg())
    st = lib.qd_decode_step(None, ctypes.byref(f.w), ctypes.byref(f.kv), 1, FAKE, None, FAKE,
                            f.pos.ctypes.data_as(POINTER(c_int32)), FAKE, None, None, None, FAKE,
                            1 << 40, None)
    _expect(st, Q.QD_EINVAL)


@pytest.mark.parametrize("over", [dict(head_dim=96), dict(hidden=60), dict(n_q_heads=5),
                                  dict(n_q_heads=18, n_kv_heads=2), dict(page_size=32),
                                  dict(n_layers=0)])
def test_bad_shapes(lib, over):
    _expect(Fixture(_cfg(**over)).decode(), Q.QD_ESHAPE)


def test_bad_dtype(lib):
    _expect(Fixture(_cfg(w_dtype=7)).decode(), Q.QD_EINVAL)


def test_batch_out_of_range(lib):
    _expect(Fixture(_cfg()).decode(batch=0), Q.QD_ESHAPE)
    _expect(Fixture(_cfg(), pos=[1] * 17, max_blocks=1).decode(), Q.QD_ESHAPE)


def test_negative_position(lib):
    _expect(Fixture(_cfg(), pos=(-1,)).decode(), Q.QD_EPOSITION)


def test_position_beyond_table(lib):
    _expect(Fixture(_cfg(), pos=(32,), max_blocks=2).decode(), Q.QD_ECAPACITY)


def test_block_table_entry_out_of_pool(lib):
    _expect(Fixture(_cfg(), pos=(20,), table=[[0, 9]], num_pages=4).decode(), Q.QD_ECAPACITY)
    _expect(Fixture(_cfg(), pos=(3,), table=[[-1, 0]], num_pages=4).decode(), Q.QD_ECAPACITY)


def test_workspace_checks(lib):
    f = Fixture(_cfg())
    _expect(f.decode(ws=None), Q.QD_EWORKSPACE)
    _expect(f.decode(ws_bytes=1024), Q.QD_EWORKSPACE)
    _expect(f.decode(ws=FAKE + 16), Q.QD_EALIGN)


def test_misaligned_weight(lib):
    f = Fixture(_cfg())
    f.layers[0].wq = FAKE + 2
    _expect(f.decode(), Q.QD_EALIGN)


def test_missing_inputs(lib):
    f = Fixture(_cfg())
    _expect(f.decode(tokens=None, x_in=None), Q.QD_EINVAL)
    _expect(f.decode(pos_host=False), Q.QD_EINVAL)
    f.layers[0].w_up = None
    _expect(f.decode(), Q.QD_EINVAL)


def test_qk_norm_needs_gains(lib):
    _expect(Fixture(_cfg(qk_norm=1)).decode(), Q.QD_EINVAL)


def test_workspace_bytes(lib):
    cfg = _cfg()
    a = Q.qd_workspace_bytes(cfg, 1, 512)
    b = Q.qd_workspace_bytes(cfg, 16, 4097)
    assert 0 < a < b
    assert Q.qd_workspace_bytes(_cfg(head_dim=96), 1, 512) == 0
    assert Q.qd_workspace_bytes(cfg, 0, 512) == 0


def test_workspace_bytes_cover_every_shorter_context(lib):
    """A workspace sized for max_ctx serves every shorter context, although a shorter
    context can take finer attention splits (more of them): the size never falls as
    max_ctx grows (batch 4, 8 KV heads of 128 dims: 2048 keys take 32 splits of 64,
    2052 take 26 of 80)."""
    cfg = _cfg(hidden=512, ffn=1024, n_q_heads=32, n_kv_heads=8, head_dim=128, vocab=1000, n_layers=2)
    for B in (1, 4, 16):
        sizes = [Q.qd_workspace_bytes(cfg, B, t) for t in range(1, 2200, 7)]
        assert all(x > 0 for x in sizes)
        assert all(u <= v for u, v in zip(sizes, sizes[1:])), B
    # and a workspace sized for a batch serves every smaller one (batch 1 adds the
    # one-launch step's buffers at the 0.5B shape)
    c05 = _cfg_05b(n_layers=2, vocab=4096)
    for t in (22, 301, 4097):
        by_batch = [Q.qd_workspace_bytes(c05, b, t) for b in range(1, 17)]
        assert all(u <= v for u, v in zip(by_batch, by_batch[1:])), t


def test_kv_append_checks(lib):
    f = Fixture(_cfg())
    ph = f.pos.ctypes.data_as(POINTER(c_int32))
    _expect(Q.qd_kv_append(f.cfg, f.kv, 3, 1, FAKE, ph, FAKE, FAKE, None), Q.QD_ESHAPE)
    _expect(Q.qd_kv_append(f.cfg, f.kv, 0, 1, FAKE, ph, None, FAKE, None), Q.QD_EINVAL)
    f2 = Fixture(_cfg(), pos=(40,))
    _expect(Q.qd_kv_append(f2.cfg, f2.kv, 0, 1, FAKE, f2.pos.ctypes.data_as(POINTER(c_int32)),
                           FAKE, FAKE, None), Q.QD_ECAPACITY)


def _prefill(f, n=10, start=0, x=FAKE, x_dtype=None, ws_bytes=1 << 40, layer_index=0):
    return Q.qd_prefill_block(f.cfg, f.layers[0], layer_index, f.kv, n, start, x,
                              Q.QD_BF16 if x_dtype is None else x_dtype, FAKE, FAKE, ws_bytes, None)


def test_prefill_checks(lib):
    f = Fixture(_cfg(), pos=(5,), max_blocks=2, num_pages=4)
    _expect(_prefill(Fixture(_cfg(w_dtype=Q.QD_F32))), Q.QD_EUNSUPPORTED)
    _expect(_prefill(f, n=0), Q.QD_ESHAPE)
    _expect(_prefill(f, start=-1), Q.QD_EPOSITION)
    _expect(_prefill(f, n=30, start=5), Q.QD_ECAPACITY)      # position 34 >= 2 pages * 16
    _expect(_prefill(f, x=None), Q.QD_EINVAL)
    _expect(_prefill(f, x_dtype=9), Q.QD_EINVAL)
    _expect(_prefill(f, ws_bytes=64), Q.QD_EWORKSPACE)
    _expect(_prefill(f, layer_index=3), Q.QD_ESHAPE)


def test_prefill_workspace_bytes(lib):
    cfg = _cfg()
    assert Q.qd_workspace_bytes(cfg, 1, 512, 512) > Q.qd_workspace_bytes(cfg, 1, 512, 16) > 0
    assert Q.qd_workspace_bytes(cfg, 1, 10, 512) == 0     # max_ctx below the prefill length


def test_int8_checks(lib):
    _expect(Fixture(_cfg(w_dtype=Q.QD_I8, hidden=72)).decode(), Q.QD_ESHAPE)      # hidden % 16
    _expect(Fixture(_cfg(w_dtype=Q.QD_I8, ffn=104)).decode(), Q.QD_ESHAPE)        # ffn % 16
    f = Fixture(_cfg(w_dtype=Q.QD_I8))
    _expect(f.decode(), Q.QD_EINVAL)                       # tokens given, s_embed NULL
    f.w.s_embed = FAKE
    _expect(f.decode(), Q.QD_EINVAL)                       # logits wanted, s_lm_head NULL
    f.w.s_lm_head = FAKE
    f.layers[0].s_up = FAKE + 2
    _expect(f.decode(), Q.QD_EINVAL)                       # misaligned row scales
    f.layers[0].s_up = None
    _expect(f.decode(), Q.QD_EINVAL)                       # missing row scales
    f2 = Fixture(_cfg(w_dtype=Q.QD_I8), pos=(3, 4))
    _expect(f2.decode(), Q.QD_EINVAL)                      # batch 2 takes int8 rows too: s_embed NULL
    f2.w.s_embed = f2.w.s_lm_head = FAKE
    _expect(f2.decode(ws_bytes=16), Q.QD_EWORKSPACE)       # ... and passes every int8 check
    _expect(_prefill(Fixture(_cfg(w_dtype=Q.QD_I8))), Q.QD_EUNSUPPORTED)


def test_quantize_checks(lib):
    _expect(Q.qd_quantize_rows_int8(None, Q.QD_BF16, 4, 32, FAKE, FAKE, None), Q.QD_EINVAL)
    _expect(Q.qd_quantize_rows_int8(FAKE, Q.QD_I8, 4, 32, FAKE, FAKE, None), Q.QD_EINVAL)
    _expect(Q.qd_quantize_rows_int8(FAKE, Q.QD_BF16, 4, 20, FAKE, FAKE, None), Q.QD_ESHAPE)
    _expect(Q.qd_quantize_rows_int8(FAKE, Q.QD_BF16, 0, 32, FAKE, FAKE, None), Q.QD_ESHAPE)
    _expect(Q.qd_quantize_rows_int8(FAKE + 8, Q.QD_F32, 4, 32, FAKE, FAKE, None), Q.QD_EALIGN)


def test_sample_checks(lib):
    s = Q.qd_sample
    _expect(s(None, 1, 100, 1.0, 10, 0.9, FAKE, FAKE, None), Q.QD_EINVAL)
    _expect(s(FAKE, 0, 100, 1.0, 10, 0.9, FAKE, FAKE, None), Q.QD_ESHAPE)
    _expect(s(FAKE, 1, 100, -1.0, 10, 0.9, FAKE, FAKE, None), Q.QD_EINVAL)
    _expect(s(FAKE, 1, 100, 1.0, 10, 0.0, FAKE, FAKE, None), Q.QD_EINVAL)
    _expect(s(FAKE, 1, 100, 1.0, 10, 1.5, FAKE, FAKE, None), Q.QD_EINVAL)
    _expect(s(FAKE, 1, 100, 1.0, 10, 0.9, None, FAKE, None), Q.QD_EINVAL)
    # top_k <= 0 or >= vocab: no top-k (top-p over the whole vocabulary), accepted;
    # 1024 < top_k < vocab: not implemented
    _expect(s(FAKE, 1, 5000, 1.0, 1025, 0.9, FAKE, FAKE, None), Q.QD_EUNSUPPORTED)
    _expect(s(FAKE, 1, 5000, 1.0, 4999, 0.9, FAKE, FAKE, None), Q.QD_EUNSUPPORTED)
    _expect(s(FAKE + 2, 1, 100, 1.0, 10, 0.9, FAKE, FAKE, None), Q.QD_EALIGN)


def test_noalloc_host_checks(lib):
    # the workspace-free step runs every host check before it touches the GPU
    f = Fixture(_cfg(vocab=300000), pos=[3] * 16, max_blocks=1)
    ph = f.pos.ctypes.data_as(POINTER(c_int32))
    need = Q.qd_workspace_bytes(f.cfg, 16, 4)
    assert need > Q.QD_NOALLOC_SCRATCH_BYTES
    _expect(Q.qd_decode_step_noalloc(f.cfg, f.w, f.kv, 16, FAKE, None, FAKE, ph, FAKE, None, None, None, None),
            Q.QD_EWORKSPACE)
    assert "static" in Q.qd_last_error()
    g = Fixture(_cfg(head_dim=96))
    _expect(Q.qd_decode_step_noalloc(g.cfg, g.w, g.kv, 1, FAKE, None, FAKE, g.pos.ctypes.data_as(POINTER(c_int32)),
                                     FAKE, None, None, None, None), Q.QD_ESHAPE)


def test_output_and_position_alignment(lib):
    f = Fixture(_cfg())
    _expect(f.decode(pos=FAKE + 2), Q.QD_EALIGN)
    _expect(f.decode(logits=FAKE + 2), Q.QD_EALIGN)
    _expect(f.decode(next_tokens=FAKE + 1), Q.QD_EALIGN)
    _expect(f.decode(x_out=FAKE + 2), Q.QD_EALIGN)
    _expect(f.decode(layer_out=FAKE + 3), Q.QD_EALIGN)
    # 4-byte aligned outputs pass the host checks (the fake workspace then fails its own)
    _expect(f.decode(logits=FAKE + 4, next_tokens=FAKE + 4, x_out=FAKE + 4, layer_out=FAKE + 4,
                     ws_bytes=16), Q.QD_EWORKSPACE)


def _cfg_05b(**over):
    return _cfg(**{**dict(n_layers=24, hidden=896, n_q_heads=14, n_kv_heads=2, head_dim=64, ffn=4864,
                          vocab=151936), **over})


def test_decode_plan_paths(lib):
    """The host plan names the kernel path a step takes."""
    p = Q.qd_decode_plan(_cfg_05b(), 1, 513)
    assert p.merge_in_o_proj == 1 and p.step_kernel == 1 and p.qkv_partials == 0
    assert p.splits * p.chunk >= 513
    # batch 16 over long contexts: the grouped matrix-core attention finishes q|k|v
    p = Q.qd_decode_plan(_cfg_05b(), 16, 4096)
    assert p.matrix_core_attention == 1 and p.qkv_partials > 1 and p.step_kernel == 0
    hd128 = _cfg(hidden=512, ffn=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, vocab=1000, n_layers=2)
    # batch 6 at 512 keys leaves too few (sequence, head, split) items: one query head
    # per workgroup on the wide kernel, no partial q|k|v
    p = Q.qd_decode_plan(hd128, 6, 512)
    assert p.heads_per_wg == 1 and p.matrix_core_attention == 0 and p.qkv_partials == 0
    # batch 8 at 1000+ keys: the grouped matrix-core kernel with partial q|k|v
    p = Q.qd_decode_plan(hd128, 8, 1001)
    assert p.matrix_core_attention == 1 and p.qkv_partials > 1
    # the step kernel takes head_dim 64, bf16 only
    assert Q.qd_decode_plan(hd128, 1, 100).step_kernel == 0
    assert Q.qd_decode_plan(_cfg_05b(kv_dtype=Q.QD_F32), 1, 100).step_kernel == 0


def test_decode_plan_fused_projection(lib, monkeypatch):
    """Batch 1 at the 0.5B shape (bf16 or int8 rows, head_dim 64, hidden <= 1024,
    no per-head norm) projects q|k|v inside the attention launch; every other
    case, and QD_FUSED_QKV=0, keeps the projection launch."""
    monkeypatch.delenv("QD_FUSED_QKV", raising=False)
    for t in (1, 144, 145, 513, 2304):
        assert Q.qd_decode_plan(_cfg_05b(), 1, t).fused_qkv == 1, t
    assert Q.qd_decode_plan(_cfg_05b(), 2, 513).fused_qkv == 0                      # batch > 1
    assert Q.qd_decode_plan(_cfg_05b(w_dtype=Q.QD_I8), 1, 513).fused_qkv == 1       # int8 rows too
    assert Q.qd_decode_plan(_cfg_05b(w_dtype=Q.QD_I8, hidden=1040), 1, 513).fused_qkv == 0  # hidden > 1024
    assert Q.qd_decode_plan(_cfg_05b(w_dtype=Q.QD_F32, kv_dtype=Q.QD_F32), 1, 100).fused_qkv == 0
    assert Q.qd_decode_plan(_cfg_05b(qk_norm=1), 1, 513).fused_qkv == 0             # per-head norm
    assert Q.qd_decode_plan(_cfg_05b(hidden=1536, ffn=8960, n_q_heads=12), 1, 513).fused_qkv == 0
    assert Q.qd_decode_plan(_cfg(hidden=512, ffn=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                 vocab=1000, n_layers=2), 1, 100).fused_qkv == 0    # head_dim 128
    monkeypatch.setenv("QD_FUSED_QKV", "0")
    assert Q.qd_decode_plan(_cfg_05b(), 1, 513).fused_qkv == 0


def test_decode_plan_o_proj_by_head_slices(lib, monkeypatch):
    """Batch 1 with a context wider than 1024 values (8B class: 32 heads of 128)
    over several splits: o_proj by head slices, no merge launch (plan value 2).
    One split, batch > 1, non-bf16 rows, QD_O_HEADS=0 and QD_DETERMINISTIC=1 keep
    the merge launch; the 0.5B shape merges inside its o_proj GEMV (value 1)."""
    monkeypatch.delenv("QD_O_HEADS", raising=False)
    monkeypatch.delenv("QD_DETERMINISTIC", raising=False)
    c8b = _cfg(hidden=4096, ffn=12288, n_q_heads=32, n_kv_heads=8, head_dim=128, vocab=151936, n_layers=36,
               qk_norm=1)
    p = Q.qd_decode_plan(c8b, 1, 4097)
    assert p.merge_in_o_proj == 2 and 1 < p.splits <= 64
    assert Q.qd_decode_plan(c8b, 1, 64).merge_in_o_proj == 0          # one split: no merge at all
    assert Q.qd_decode_plan(c8b, 2, 4097).merge_in_o_proj == 0        # batch 2
    assert Q.qd_decode_plan(_cfg_05b(), 1, 513).merge_in_o_proj == 1
    for name, val in (("QD_O_HEADS", "0"), ("QD_DETERMINISTIC", "1")):
        monkeypatch.setenv(name, val)
        assert Q.qd_decode_plan(c8b, 1, 4097).merge_in_o_proj == 0, name
        monkeypatch.delenv(name)
    assert Q.qd_decode_plan(c8b, 1, 4097).merge_in_o_proj == 2


def test_decode_plan_checks(lib):
    out = Q.qd_decode_plan_info()
    _expect(lib.qd_decode_plan(_cfg_05b(), 1, 10, None), Q.QD_EINVAL)
    _expect(lib.qd_decode_plan(_cfg_05b(), 0, 10, ctypes.byref(out)), Q.QD_ESHAPE)
    _expect(lib.qd_decode_plan(_cfg_05b(), 1, 0, ctypes.byref(out)), Q.QD_ESHAPE)
    _expect(lib.qd_decode_plan(_cfg_05b(), 1, 1 << 24, ctypes.byref(out)), Q.QD_ECAPACITY)
    _expect(lib.qd_decode_plan(_cfg(head_dim=96), 1, 10, ctypes.byref(out)), Q.QD_ESHAPE)
