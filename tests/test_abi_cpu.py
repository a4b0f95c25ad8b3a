"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call
(no compute runs here; the device pointers given are never dereferenced)."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


@pytest.fixture(scope="module")
def dsp():
    import block_draft_model_dspark_amd as dsp
    if not os.path.exists(dsp.LIB_PATH):
        from block_draft_model_dspark_amd import build
        build.build()
    dsp.load_library()
    return dsp


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dspark_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree(dsp):
    decl = declared_functions()
    assert set(decl) == set(dsp.EXPORTED), decl


def test_every_declared_symbol_is_exported(dsp):
    lib = ctypes.CDLL(dsp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


FAKE = 0x10000  # never dereferenced: all paths below fail validation first


def fake_table(dsp, cfg, drop=None, bad_shape=None):
    names = synth.tensor_names(cfg, with_fc=False)
    table = (dsp.Weight * len(names))()
    keep = []
    n = 0
    for name in names:
        if name == drop:
            continue
        shape = list(synth.tensor_shape(cfg, name))
        if name == bad_shape:
            shape[0] += 16
        kind = cfg.weight_dtype if synth.gen.is_matrix(name) else cfg.act_dtype
        b = name.encode()
        keep.append(b)
        table[n].name = b
        table[n].dtype = {"f32": 0, "bf16": 1, "q4": 2}[kind]
        table[n].data = FAKE
        table[n].scales = FAKE
        table[n].biases = FAKE
        table[n].rows = shape[0]
        table[n].cols = shape[1] if len(shape) > 1 else 1
        n += 1
    return table, n, keep


def make_config(dsp, cfg, **over):
    c = dsp.Config()
    for f, _ in dsp.Config._fields_:
        if hasattr(cfg, f) and getattr(cfg, f) is not None and not isinstance(getattr(cfg, f), str):
            setattr(c, f, getattr(cfg, f))
    c.attention_k_eq_v = 1
    c.markov_head_vanilla = 1
    c.activation_gelu_tanh = 1
    c.fc_in = 0
    c.final_logit_softcapping = cfg.final_logit_softcapping or 0.0
    c.weight_dtype = {"f32": 0, "bf16": 1, "q4": 2}[cfg.weight_dtype]
    c.act_dtype = {"f32": 0, "bf16": 1, "q4": 2}[cfg.act_dtype]
    for k, v in over.items():
        setattr(c, k, v)
    return c


def create(dsp, c, table, n):
    h = ctypes.c_void_p()
    st = dsp._lib.dspark_model_create(ctypes.byref(c), table, n, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("field,value,status", [
    ("attention_k_eq_v", 0, 3), ("markov_head_vanilla", 0, 3), ("activation_gelu_tanh", 0, 3),
    ("global_head_dim", 96, 3), ("num_global_key_value_heads", 3, 2), ("block_size", 0, 1),
    ("mask_token_id", 5000, 1), ("vocab_size", 1000, 3), ("vocab_size", (1 << 22) + 64, 3)])
def test_config_guards(dsp, field, value, status):
    cfg = synth.TINY
    table, n, keep = fake_table(dsp, cfg)
    c = make_config(dsp, cfg, **{field: value})
    st, _ = create(dsp, c, table, n)
    assert st == status, dsp._lib.dspark_last_error()
    assert dsp._lib.dspark_last_error()


def test_missing_and_misshapen_tensors(dsp):
    cfg = synth.TINY
    c = make_config(dsp, cfg)
    table, n, keep = fake_table(dsp, cfg, drop="layers.0.mlp.up_proj.weight")
    st, _ = create(dsp, c, table, n)
    assert st == 2 and b"up_proj" in dsp._lib.dspark_last_error()
    table, n, keep = fake_table(dsp, cfg, bad_shape="lm_head.weight")
    st, _ = create(dsp, c, table, n)
    assert st == 2 and b"lm_head" in dsp._lib.dspark_last_error()


def test_draft_rows_host_validation(dsp):
    """A model over fake pointers validates calls without touching the GPU."""
    cfg = synth.TINY
    c = make_config(dsp, cfg)
    table, n, keep = fake_table(dsp, cfg)
    st, h = create(dsp, c, table, n)
    assert st == 0
    lib = dsp._lib
    P = ctypes.c_void_p
    kp = (P * 1)(FAKE)
    lens = (ctypes.c_int32 * 1)(32)
    pos = (ctypes.c_int32 * 1)(32)
    ws_need = lib.dspark_draft_workspace_bytes(h, 1, 32, 32)
    assert ws_need > 0

    def call(anchor=5, A=1, ws=ws_need, ws_ptr=FAKE * 16, aux=FAKE, tok=FAKE):
        anc = (ctypes.c_int32 * 1)(anchor)
        return lib.dspark_draft_rows(h, A, kp, kp, lens, anc, pos, tok, None, aux, ws_ptr, ws, None)

    assert call(anchor=-1) == 1
    assert call(anchor=cfg.V) == 1
    assert call(A=0) == 1
    assert call(A=65) == 3
    assert call(ws=ws_need - 1) == 4
    assert call(ws_ptr=FAKE * 16 + 8) == 4
    assert call(aux=None) == 1
    assert call(tok=None) == 1
    bad_lens = (ctypes.c_int32 * 1)(-1)
    anc = (ctypes.c_int32 * 1)(5)
    assert lib.dspark_draft_rows(h, 1, kp, kp, bad_lens, anc, pos, FAKE, None, FAKE, FAKE * 16, ws_need, None) == 1
    nullk = (P * 1)(None)
    assert lib.dspark_draft_rows(h, 1, nullk, nullk, lens, anc, pos, FAKE, None, FAKE, FAKE * 16, ws_need, None) == 1
    # projection
    n_ws = lib.dspark_project_workspace_bytes(h, 0, 1, 32)
    p0 = (ctypes.c_int32 * 1)(-3)
    outs = (P * 1)(FAKE)
    assert lib.dspark_project_context_kv(h, 0, FAKE, 1, 32, p0, outs, outs, FAKE * 16, n_ws, None) == 1
    p0[0] = 0
    assert lib.dspark_project_context_kv(h, 1, FAKE, 1, 32, p0, outs, outs, FAKE * 16, n_ws, None) == 3  # no fc
    assert lib.dspark_project_context_kv(h, 0, FAKE, 1, 32, p0, outs, outs, FAKE * 16, n_ws - 1, None) == 4
    assert lib.dspark_project_context_kv(h, 7, FAKE, 1, 32, p0, outs, outs, FAKE * 16, n_ws, None) == 1
    lib.dspark_model_destroy(h)


@pytest.mark.parametrize("gx,gy", [(1, 1), (3, 5), (8, 1), (8, 8), (16, 4), (256, 4), (16, 64), (8, 64),
                                   (36, 16), (12, 24), (24, 16), (7, 9), (64, 8), (128, 128)])
def test_tall_tile_order_is_a_bijection(dsp, gx, gy):
    """The tiled GEMM's XCD-aware renumbering covers every output tile once
    (for the grid shapes of the round and the projection and odd ones)."""
    lib = dsp._lib
    bx, by = ctypes.c_int(), ctypes.c_int()
    seen = set()
    for w in range(gx * gy):
        assert lib.dspark_tall_tile_of(gx, gy, w, ctypes.byref(bx), ctypes.byref(by)) == 0
        assert 0 <= bx.value < gx and 0 <= by.value < gy
        seen.add((bx.value, by.value))
    assert len(seen) == gx * gy
    assert lib.dspark_tall_tile_of(gx, gy, gx * gy, ctypes.byref(bx), ctypes.byref(by)) == 1


def test_tall_tile_order_keeps_a_row_tile_on_one_xcd(dsp):
    """More than 8 row tiles: every tile of row tile r runs on XCD r mod 8
    (workgroup w on XCD w mod 8), so an activation row is fetched by one L2."""
    lib = dsp._lib
    bx, by = ctypes.c_int(), ctypes.c_int()
    for gx, gy in [(16, 64), (8, 64), (12, 24)]:
        for w in range(gx * gy):
            lib.dspark_tall_tile_of(gx, gy, w, ctypes.byref(bx), ctypes.byref(by))
            assert by.value % 8 == w % 8


@pytest.mark.parametrize("gx,S,R", [(2048, 1, 4), (16, 1, 16), (512, 1, 4), (36, 8, 1), (36, 8, 2), (32, 8, 2),
                                    (8, 1, 3), (12, 1, 4), (64, 1, 2), (256, 1, 1), (24, 2, 5), (32, 3, 3), (7, 3, 2)])
def test_stream_block_order_is_a_bijection(dsp, gx, S, R):
    """The weight-streaming GEMM's renumbering covers every (column block,
    K slice, row block) once; with several row blocks and gx * S a multiple
    of 8, the row blocks of a (column block, slice) share one XCD (workgroup
    x + gx (y + S z) on XCD (x + gx (y + S z)) mod 8) and follow each other
    in launch order."""
    lib = dsp._lib
    bx, by, bz = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    seen, where = set(), {}
    for z in range(R):
        for y in range(S):
            for x in range(gx):
                assert lib.dspark_stream_block_of(gx, S, R, x, y, z, ctypes.byref(bx), ctypes.byref(by),
                                                  ctypes.byref(bz)) == 0
                assert 0 <= bx.value < gx and 0 <= by.value < S and 0 <= bz.value < R
                seen.add((bx.value, by.value, bz.value))
                where.setdefault((bx.value, by.value), []).append(x + gx * (y + S * z))
    assert len(seen) == gx * S * R
    if R > 1 and (gx * S) % 8 == 0:
        for ws in where.values():
            assert len({w % 8 for w in ws}) == 1
            assert max(ws) - min(ws) == 8 * (R - 1)
    else:
        assert all(ws == [u[0] + gx * (u[1] + S * z) for z in range(R)] for u, ws in where.items())
    assert lib.dspark_stream_block_of(gx, S, R, gx, 0, 0, ctypes.byref(bx), ctypes.byref(by), ctypes.byref(bz)) == 1


def test_draft_workspace_scales_with_context_up_to_the_split_cap(dsp):
    """Only the attention partials scale with the contexts: at most
    min(512, ceil(total / 32)) + 2A splits, so the size grows with total_ctx
    and stops growing once 512 context splits are reached."""
    cfg = synth.FULL
    c = make_config(dsp, cfg)
    table, n, keep = fake_table(dsp, cfg)
    st, h = create(dsp, c, table, n)
    assert st == 0
    f = dsp._lib.dspark_draft_workspace_bytes
    sizes = [f(h, 2, t, t) for t in (0, 32, 512, 4096, 16384, 32768, 65536)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes) and sizes[1] > sizes[0]
    assert sizes[-1] == sizes[-2] == f(h, 2, 10 ** 6, 10 ** 6)  # >= 512 * 32 keys: capped
    assert f(h, 2, 100, 201) == 0 and f(h, 2, -1, 0) == 0 and f(h, 0, 10, 10) == 0
    dsp._lib.dspark_model_destroy(h)


def test_confidence_head_guards(dsp):
    base = synth.scaled(synth.TINY, enable_confidence_head=True, confidence_head_with_markov=True)
    table, n, keep = fake_table(dsp, base)
    st, h = create(dsp, make_config(dsp, base), table, n)
    assert st == 0, dsp._lib.dspark_last_error()
    dsp._lib.dspark_model_destroy(h)
    # the Markov feature needs a Markov head
    st, _ = create(dsp, make_config(dsp, base, markov_rank=0), table, n)
    assert st == 1 and b"markov" in dsp._lib.dspark_last_error()
    # a missing head tensor
    table, n, keep = fake_table(dsp, base, drop="confidence_head.proj.bias")
    st, _ = create(dsp, make_config(dsp, base), table, n)
    assert st == 2 and b"confidence_head" in dsp._lib.dspark_last_error()
    # confidences requested from a model without the head
    plain = synth.TINY
    table, n, keep = fake_table(dsp, plain)
    st, h = create(dsp, make_config(dsp, plain), table, n)
    assert st == 0
    P = ctypes.c_void_p
    kp = (P * 1)(FAKE)
    one = (ctypes.c_int32 * 1)(32)
    anc = (ctypes.c_int32 * 1)(5)
    ws = dsp._lib.dspark_draft_workspace_bytes(h, 1, 32, 32)
    assert dsp._lib.dspark_draft_rows_conf(h, 1, kp, kp, one, anc, one, None, FAKE, None, FAKE, None, FAKE,
                                           FAKE * 16, ws, None) == 1
    dsp._lib.dspark_model_destroy(h)


def test_rnn_head_guards(dsp):
    base = synth.scaled(synth.TINY, markov_head_type="rnn")
    table, n, keep = fake_table(dsp, base)
    st, h = create(dsp, make_config(dsp, base, markov_head_vanilla=0, markov_head_rnn=1), table, n)
    assert st == 0, dsp._lib.dspark_last_error()
    dsp._lib.dspark_model_destroy(h)
    # both head kinds at once, and a head that is neither (the gated one)
    st, _ = create(dsp, make_config(dsp, base, markov_head_vanilla=1, markov_head_rnn=1), table, n)
    assert st == 1
    st, _ = create(dsp, make_config(dsp, base, markov_head_vanilla=0, markov_head_rnn=0), table, n)
    assert st == 3
    table, n, keep = fake_table(dsp, base, drop="markov_head.rnn_wh.weight")
    st, _ = create(dsp, make_config(dsp, base, markov_head_vanilla=0, markov_head_rnn=1), table, n)
    assert st == 2 and b"rnn_wh" in dsp._lib.dspark_last_error()
