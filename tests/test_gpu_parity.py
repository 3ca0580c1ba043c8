"""GPU parity of the HIP path against the CPU float64 oracle (needs gfx950).

Every case draws seeded inputs, runs the library through the C ABI (via the
ctypes binding), and compares with the oracle on the same stored values:
element by element at sizes the oracle finishes quickly (several tiles and
a ragged tail), and on shapes that give the persistent grids more work
items than compute units. The five benchmark configurations are checked
element by element in test_gpu_configs.py.
"""

import numpy as np
import pytest

import oracle
from tests.helpers import assert_bf16_parity, assert_f32_parity, to_dev, to_np
from tiled_attention_12_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def ta(lib_path):
    import tiled_attention_12_amd as ta
    return ta


def _vals(x, names):
    return [inputs.stored_values(x[n]) for n in names]


@pytest.fixture(params=[4, 8], ids=["waves4", "waves8"])
def dense_waves(request, monkeypatch):
    """Forces the dense prefill's workgroup shape (4 waves x 128 rows, two per
    CU, or 8 waves x 256 rows); unset, the launcher picks it from the launch
    size, and small test shapes would only reach the 4-wave one."""
    monkeypatch.setenv("TATTN_MHA_WAVES", str(request.param))
    return request.param


def _run_mha(ta, dev, x, causal, scale, fp32=False):
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    fn = ta.attn_fwd_f32 if fp32 else ta.attn_fwd
    o, lse = fn(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


# ------------------------------------------------------------------ fp32 path

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,skv", [(1, 1), (33, 70), (130, 130), (64, 200), (200, 64)])
def test_fp32_shapes(ta, dev, D, causal, sq, skv):
    x = inputs.mha_inputs(2, 2, sq, skv, D, seed=100 + sq + skv + D, dtype="f32")
    scale = float(np.float32(D ** -0.5))
    o, lse = _run_mha(ta, dev, x, causal, scale, fp32=True)
    ro, rl = oracle.attention(x["q"], x["k"], x["v"], scale, causal=causal)
    assert_f32_parity(o, lse, ro, rl, f"fp32 D={D} causal={causal} {sq}x{skv}")


# ------------------------------------------------------------------ bf16 prefill

SHAPES = [(1, 1), (7, 7), (63, 63), (64, 64), (65, 65), (127, 129), (129, 127), (200, 257),
          (256, 256), (300, 300), (5, 300), (300, 5), (130, 1000)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("sq,skv", SHAPES)
def test_bf16_shapes(ta, dev, D, causal, sq, skv, dense_waves):
    x = inputs.mha_inputs(2, 3, sq, skv, D, seed=7 * sq + skv + D + int(causal))
    scale = float(np.float32(D ** -0.5))
    o, lse = _run_mha(ta, dev, x, causal, scale)
    ro, rl = oracle.attention(*_vals(x, "qkv"), scale, causal=causal)
    assert_bf16_parity(o, lse, ro, rl, f"bf16 D={D} causal={causal} {sq}x{skv}")


def test_bf16_empty_keys_and_fully_masked_rows(ta, dev, dense_waves):
    x = inputs.mha_inputs(1, 2, 40, 0, 128, seed=3)
    q = to_dev(x["q"], dev)
    kv = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    o, lse = ta.attn_fwd(q, kv, kv)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    # Sq > Skv causal: the first Sq - Skv rows see nothing
    x = inputs.mha_inputs(1, 2, 150, 20, 64, seed=4)
    o, lse = _run_mha(ta, dev, x, True, 0.125)
    ro, rl = oracle.attention(*_vals(x, "qkv"), 0.125, causal=True)
    assert np.all(o[:, :, :130] == 0) and np.all(np.isneginf(lse[:, :, :130]))
    assert_bf16_parity(o, lse, ro, rl, "Sq > Skv causal")


def test_bf16_single_and_identical_keys(ta, dev):
    x = inputs.mha_inputs(1, 2, 100, 1, 128, seed=5)
    o, lse = _run_mha(ta, dev, x, False, 0.1)
    v = inputs.stored_values(x["v"]).astype(np.float64)
    assert np.array_equal(o, np.broadcast_to(v, o.shape))
    ro, rl = oracle.attention(*_vals(x, "qkv"), 0.1)
    assert np.abs(lse - rl).max() <= 1e-3
    x = inputs.mha_inputs(1, 2, 70, 150, 64, seed=6)
    x["k"][:] = x["k"][:, :, :1]
    o, lse = _run_mha(ta, dev, x, False, 0.1)
    v = inputs.stored_values(x["v"]).astype(np.float64)
    assert np.abs(o - v.mean(axis=2, keepdims=True)).max() <= 1e-2
    ro, rl = oracle.attention(*_vals(x, "qkv"), 0.1)
    assert np.abs(lse - rl).max() <= 1e-3


def test_bf16_causal_row0_and_future_keys(ta, dev, dense_waves):
    x = inputs.mha_inputs(2, 2, 333, 333, 128, seed=11)
    o1, l1 = _run_mha(ta, dev, x, True, 0.09)
    v = inputs.stored_values(x["v"]).astype(np.float64)
    assert np.array_equal(o1[:, :, 0], v[:, :, 0])
    y = {n: x[n].copy() for n in "qkv"}
    y["k"][:, :, 200:] = inputs.f32_to_bf16_bits(np.float32(2.0) * inputs.stored_values(y["k"][:, :, 200:]))
    y["v"][:, :, 200:] = inputs.f32_to_bf16_bits(np.float32(-3.0) * inputs.stored_values(y["v"][:, :, 200:]))
    o2, l2 = _run_mha(ta, dev, y, True, 0.09)
    assert np.array_equal(o1[:, :, :200], o2[:, :, :200])
    assert np.array_equal(l1[:, :, :200], l2[:, :, :200])


def test_bf16_row_shift_invariance(ta, dev):
    # a key column of ones plus a per-row query entry adds a constant to each score row
    x = inputs.mha_inputs(1, 1, 96, 160, 64, seed=12)
    q = inputs.stored_values(x["q"]).copy()
    k = inputs.stored_values(x["k"]).copy()
    k[..., 0] = 1.0
    q[..., 0] = 0.0
    base = {"q": inputs.f32_to_bf16_bits(q), "k": inputs.f32_to_bf16_bits(k), "v": x["v"]}
    shift = q.copy()
    shift[..., 0] = np.linspace(-8, 8, 96, dtype=np.float32).reshape(1, 1, 96)
    moved = dict(base, q=inputs.f32_to_bf16_bits(shift))
    o1, l1 = _run_mha(ta, dev, base, False, 0.125)
    o2, l2 = _run_mha(ta, dev, moved, False, 0.125)
    c = 0.125 * inputs.stored_values(moved["q"])[..., 0].astype(np.float64)
    assert np.abs(o1 - o2).max() <= 1e-2
    assert np.abs((l2 - l1) - c).max() <= 2e-3


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_key_permutation_invariance(ta, dev, D):
    # non-causal attention is a sum over keys: permuting K and V rows together
    # (across tiles and the ragged tail) changes O only by rounding order
    x = inputs.mha_inputs(2, 3, 200, 333, D, seed=14)
    perm = np.random.default_rng(15).permutation(333)
    moved = dict(x, k=np.ascontiguousarray(x["k"][:, :, perm]), v=np.ascontiguousarray(x["v"][:, :, perm]))
    o1, l1 = _run_mha(ta, dev, x, False, 0.1)
    o2, l2 = _run_mha(ta, dev, moved, False, 0.1)
    assert np.abs(o1 - o2).max() <= 1e-2
    assert np.abs(l1 - l2).max() <= 1e-3
    assert np.linalg.norm(o1 - o2) <= 1e-2 * np.linalg.norm(o1)


def test_bf16_deterministic(ta, dev):
    x = inputs.mha_inputs(2, 4, 300, 300, 128, seed=13)
    a = _run_mha(ta, dev, x, True, 0.088)
    b = _run_mha(ta, dev, x, True, 0.088)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("causal", [False, True])
def test_dense_shape_choice_follows_the_launch_size(ta, dev, causal, monkeypatch):
    # unforced, a launch with few 256-row items runs the 4-wave shape and a
    # launch with at least one item per CU the 8-wave shape: the automatic
    # result is bitwise the forced one (both shapes compute each row alike,
    # but which tiles a shape masks can change the rounding, so the two shapes
    # are compared with the oracle, not with each other)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    D = 128
    cases = [(1, 2, 700, 4)]  # 2 * 3 items of 256 rows
    big_h = -(-cus // 4)  # 4 items of 256 rows per head: at least one item per CU
    cases.append((1, big_h, 1024, 8))
    for B, H, S, expect in cases:
        x = inputs.mha_inputs(B, H, S, S, D, seed=90 + H)
        monkeypatch.delenv("TATTN_MHA_WAVES", raising=False)
        auto = _run_mha(ta, dev, x, causal, 0.088)
        monkeypatch.setenv("TATTN_MHA_WAVES", str(expect))
        forced = _run_mha(ta, dev, x, causal, 0.088)
        assert np.array_equal(auto[0], forced[0]) and np.array_equal(auto[1], forced[1]), (B, H, S, expect)
    monkeypatch.delenv("TATTN_MHA_WAVES")


@pytest.mark.parametrize("causal", [False, True])
def test_dense_shapes_with_more_items_than_workgroup_slots(ta, dev, causal, dense_waves):
    # 4 x 16 heads of 1100 rows: 576 items of 128 rows (more than two per CU
    # at 256 CUs) or 320 of 256; outputs start as NaN so a skipped or
    # mis-mapped item fails, and every element is checked
    B, H, S, D = 4, 16, 1100, 128
    x = inputs.mha_inputs(B, H, S, S, D, seed=93 + int(causal))
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    o = torch.full((B, H, S, D), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=dev)
    ta.attn_fwd(q, k, v, causal=causal, scale=0.088, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(*_vals(x, "qkv"), 0.088, causal=causal)
    assert_bf16_parity(to_np(o), to_np(lse), ro, rl, f"{dense_waves} waves, {B}x{H}x{S} causal={causal}")


# ------------------------------------------------------------------ MLA decode

def _run_mla(ta, dev, m, scale, fn="mla_decode"):
    args = [to_dev(m[n], dev) for n in ("q", "q_pe", "kv", "k_pe")]
    o, lse = getattr(ta, fn)(*args, to_dev(m["indptr"], dev), scale)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


def _mla_vals(m):
    return [inputs.stored_values(m[n]) for n in ("q", "q_pe", "kv", "k_pe")]


@pytest.mark.parametrize("H", [32, 64, 128])
@pytest.mark.parametrize("lens", [[1], [31, 32, 33], [0, 5, 0, 64, 1], [500, 1, 77], [0, 0]])
def test_mla_small(ta, dev, H, lens):
    B = len(lens)
    rng = np.random.default_rng(sum(lens) + H)
    m = inputs.mla_inputs(B, H, seed=int(rng.integers(1 << 30)), kv_len=1)
    # rebuild with the requested lengths (same generator recipe, explicit lengths)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(indptr[-1])
    g = np.random.default_rng(int(rng.integers(1 << 30)))
    m["kv"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 512), dtype=np.float32) * np.float32(0.3))
    m["k_pe"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 64), dtype=np.float32) * np.float32(0.3))
    m["indptr"] = indptr
    if n == 0:
        m["kv"] = np.zeros((1, 512), np.uint16)
        m["k_pe"] = np.zeros((1, 64), np.uint16)
    scale = float(np.float32(576 ** -0.5))
    o, lse = _run_mla(ta, dev, m, scale)
    ro, rl = oracle.mla_decode(*_mla_vals(m), indptr, scale)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
    assert_bf16_parity(o, lse, ro, rl, f"mla H={H} lens={lens}")


@pytest.mark.parametrize("fn", ["mla_decode", "mla_decode_noalloc"])
@pytest.mark.parametrize("H", [1, 16, 33, 48, 96, 100, 127])
def test_mla_any_head_count(ta, dev, H, fn):
    # head counts that are not a multiple of 32: the last wave carries padding
    # heads whose results must not reach O, LSE or the neighbouring partials
    lens = [1, 300, 0, 2049, 64]
    m = _ragged_mla(dev, lens, H, seed=50 + H)
    scale = float(np.float32(576 ** -0.5))
    o, lse = _run_mla(ta, dev, m, scale, fn=fn)
    ro, rl = oracle.mla_decode(*_mla_vals(m), m["indptr"], scale)
    assert o.shape == (len(lens), H, 512) and lse.shape == (len(lens), H)
    assert np.all(o[2] == 0) and np.all(np.isneginf(lse[2]))
    assert_bf16_parity(o, lse, ro, rl, f"{fn} H={H}")


def test_mla_ragged_batch_equals_standalone(ta, dev):
    lens = [700, 3000, 129, 4097]
    m = inputs.mla_inputs(len(lens), 128, seed=21, kv_len=1)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = np.random.default_rng(22)
    n = int(indptr[-1])
    m["kv"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 512), dtype=np.float32) * np.float32(0.3))
    m["k_pe"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 64), dtype=np.float32) * np.float32(0.3))
    m["indptr"] = indptr
    scale = float(np.float32(576 ** -0.5))
    o, lse = _run_mla(ta, dev, m, scale)
    b = 3
    one = {"q": m["q"][b:b + 1], "q_pe": m["q_pe"][b:b + 1], "kv": m["kv"][indptr[b]:indptr[b + 1]],
           "k_pe": m["k_pe"][indptr[b]:indptr[b + 1]], "indptr": np.array([0, lens[b]], np.int32)}
    o1, l1 = _run_mla(ta, dev, one, scale)
    assert np.abs(o[b] - o1[0]).max() <= 1e-2 and np.abs(lse[b] - l1[0]).max() <= 1e-3
    ro, rl = oracle.mla_decode(*_mla_vals(m), indptr, scale)
    assert_bf16_parity(o, lse, ro, rl, "mla ragged 4")


@pytest.mark.parametrize("H", [32, 128])
@pytest.mark.parametrize("B", [1023, 1100])
def test_mla_many_batches(ta, dev, B, H):
    # below 1024 batches the split kernel forms the tile prefix itself; from
    # 1024 on a separate plan launch does: both paths, with empty batches
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 4, size=B)
    lens[::7] = 0
    m = inputs.mla_inputs(B, H, seed=B + 1, kv_len=1)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(indptr[-1])
    g = np.random.default_rng(B + 2)
    m["kv"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 512), dtype=np.float32) * np.float32(0.3))
    m["k_pe"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 64), dtype=np.float32) * np.float32(0.3))
    m["indptr"] = indptr
    scale = float(np.float32(576 ** -0.5))
    o, lse = _run_mla(ta, dev, m, scale)
    ro, rl = oracle.mla_decode(*_mla_vals(m), indptr, scale)
    empty = lens == 0
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    assert_bf16_parity(o, lse, ro, rl, f"mla B={B} H={H}")


def test_mla_key_permutation_invariance(ta, dev):
    # permuting each batch's key rows (latent and rotary together) moves keys
    # across tiles, splits and the ragged tail; O changes only by rounding
    lens = [700, 1500, 33]
    m = inputs.mla_inputs(len(lens), 128, seed=24, kv_len=1)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = np.random.default_rng(25)
    n = int(indptr[-1])
    m["kv"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 512), dtype=np.float32) * np.float32(0.3))
    m["k_pe"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 64), dtype=np.float32) * np.float32(0.3))
    m["indptr"] = indptr
    perm = np.concatenate([indptr[b] + g.permutation(L) for b, L in enumerate(lens)])
    moved = dict(m, kv=np.ascontiguousarray(m["kv"][perm]), k_pe=np.ascontiguousarray(m["k_pe"][perm]))
    scale = float(np.float32(576 ** -0.5))
    o1, l1 = _run_mla(ta, dev, m, scale)
    o2, l2 = _run_mla(ta, dev, moved, scale)
    assert np.abs(o1 - o2).max() <= 1e-2
    assert np.abs(l1 - l2).max() <= 1e-3
    assert np.linalg.norm(o1 - o2) <= 1e-2 * np.linalg.norm(o1)


def test_mla_deterministic(ta, dev):
    m = inputs.mla_inputs(8, 128, seed=23, kv_len_range=(1, 3000))
    scale = float(np.float32(576 ** -0.5))
    a = _run_mla(ta, dev, m, scale)
    b = _run_mla(ta, dev, m, scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _mla_dev_inputs(dev, B, H, seed, kv_len_range):
    m = inputs.mla_inputs(B, H, seed=seed, kv_len_range=kv_len_range)
    args = [to_dev(m[n], dev) for n in ("q", "q_pe", "kv", "k_pe")] + [to_dev(m["indptr"], dev)]
    return m, args


def test_mla_workspace_grows_and_is_reused(ta, dev):
    # the library's decode workspace grows to the largest call and is reused;
    # calls enqueued back to back without a synchronisation in between must
    # each see their own partials
    scale = float(np.float32(576 ** -0.5))
    small, sa = _mla_dev_inputs(dev, 2, 128, 31, (1, 900))
    big, ba = _mla_dev_inputs(dev, 600, 32, 32, (1, 40))
    o1, l1 = ta.mla_decode(*sa, scale)
    o2, l2 = ta.mla_decode(*ba, scale)  # needs a larger workspace
    o3, l3 = ta.mla_decode(*sa, scale)
    o4, l4 = ta.mla_decode(*ba, scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert torch.equal(o2, o4) and torch.equal(l2, l4)
    ro, rl = oracle.mla_decode(*_mla_vals(small), small["indptr"], scale)
    assert_bf16_parity(to_np(o1), to_np(l1), ro, rl, "mla small after growth")
    ro, rl = oracle.mla_decode(*_mla_vals(big), big["indptr"], scale)
    assert_bf16_parity(to_np(o2), to_np(l2), ro, rl, "mla big")


def test_mla_calls_on_two_streams(ta, dev):
    # calls on two streams share the device's workspace one after another
    scale = float(np.float32(576 ** -0.5))
    ma, aa = _mla_dev_inputs(dev, 16, 128, 33, (1, 2000))
    mb, ab = _mla_dev_inputs(dev, 9, 64, 34, (1, 3000))
    ra = ta.mla_decode(*aa, scale)
    rb = ta.mla_decode(*ab, scale)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    outs = []
    for rep in range(3):
        with torch.cuda.stream(s1):
            xa = ta.mla_decode(*aa, scale)
        with torch.cuda.stream(s2):
            xb = ta.mla_decode(*ab, scale)
        outs.append((xa, xb))
    torch.cuda.synchronize()
    for xa, xb in outs:
        assert torch.equal(xa[0], ra[0]) and torch.equal(xa[1], ra[1])
        assert torch.equal(xb[0], rb[0]) and torch.equal(xb[1], rb[1])
    ro, rl = oracle.mla_decode(*_mla_vals(mb), mb["indptr"], scale)
    assert_bf16_parity(to_np(rb[0]), to_np(rb[1]), ro, rl, "mla stream b")


def test_mla_streams_beyond_the_workspace_slots(ta, dev):
    # each stream of a device gets its own decode workspace, up to eight; more
    # streams take over the least recently used one. Ten streams, each with
    # growing calls back to back and no synchronisation in between, must all
    # get the results of a lone call.
    scale = float(np.float32(576 ** -0.5))
    cases = [_mla_dev_inputs(dev, 3 + 7 * i, 128 if i % 2 else 64, 60 + i, (1, 300 + 200 * i)) for i in range(10)]
    ref = []
    for m, args in cases:
        ref.append(ta.mla_decode(*args, scale))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(dev) for _ in range(10)]
    got = []
    for rep in range(2):
        for i, (s, (m, args)) in enumerate(zip(streams, cases)):
            with torch.cuda.stream(s):
                got.append((i, ta.mla_decode(*args, scale)))
    torch.cuda.synchronize()
    for i, (o, l) in got:
        assert torch.equal(o, ref[i][0]) and torch.equal(l, ref[i][1]), f"stream {i}"
    m, _ = cases[3]
    ro, rl = oracle.mla_decode(*_mla_vals(m), m["indptr"], scale)
    assert_bf16_parity(to_np(ref[3][0]), to_np(ref[3][1]), ro, rl, "mla stream case 3")


_TAKEOVER_SCRIPT = r"""
import numpy as np, torch
import tiled_attention_12_amd as ta
from tiled_attention_12_amd import inputs
dev = torch.device("cuda:0")
scale = float(np.float32(576 ** -0.5))
cases = []
for i in range(9):
    m = inputs.mla_inputs(2 + 3 * i, 64, seed=300 + i, kv_len_range=(1, 400 + 150 * i))
    args = [torch.from_numpy(np.ascontiguousarray(m[k]).view(np.int16)).view(torch.bfloat16).to(dev)
            for k in ("q", "q_pe", "kv", "k_pe")] + [torch.from_numpy(m["indptr"]).to(dev)]
    cases.append(args)
streams = [torch.cuda.Stream(dev) for _ in range(9)]
# stream 0 is the only stream with a workspace at its call: no event is kept
with torch.cuda.stream(streams[0]):
    first = ta.mla_decode(*cases[0], scale)
torch.cuda.synchronize()
ref = [ta.mla_decode(*c, scale) for c in cases]  # lone calls (default stream: a second workspace)
torch.cuda.synchronize()
got = []
for i in range(1, 9):  # streams 1..7 take the six free workspaces and then the least recently used
    with torch.cuda.stream(streams[i]):
        got.append((i, ta.mla_decode(*cases[i], scale)))
with torch.cuda.stream(streams[0]):
    got.append((0, ta.mla_decode(*cases[0], scale)))
torch.cuda.synchronize()
assert torch.equal(first[0], ref[0][0]) and torch.equal(first[1], ref[0][1])
for i, (o, l) in got:
    assert torch.equal(o, ref[i][0]) and torch.equal(l, ref[i][1]), i
print("takeover ok", flush=True)
"""


def test_mla_workspace_takeover_after_single_stream_use(lib_path):
    # In a fresh process: a stream's workspace whose last call came while it
    # was the only stream with one (no completion event kept) is taken over
    # by another stream once every workspace is in use; the takeover waits
    # for the device on the host, and every call still gets a lone call's
    # results. (8 workspaces per device: stream 0, the default stream and
    # streams 1..6 fill them, stream 7 takes over stream 0's, stream 8 the
    # next least recently used, then stream 0 takes one back.)
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", _TAKEOVER_SCRIPT], capture_output=True, text=True, timeout=300,
                       cwd=root, env=env)
    assert r.returncode == 0 and "takeover ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]


@pytest.mark.parametrize("causal", [False, True])
def test_more_items_than_compute_units_without_xcd_order(ta, dev, causal):
    # B*H = 5 is not a multiple of 8, so items are taken in plain order; 5 heads
    # of 64 query tiles are 320 items, more than one pass of a 256-CU grid.
    # Every row block of a few heads is checked on sampled rows.
    B, H, S, D = 1, 5, 16384, 128
    x = inputs.mha_inputs(B, H, S, S, D, seed=77)
    o, lse = _run_mha(ta, dev, x, causal, 0.088)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(78)
    rows = np.unique(np.concatenate([np.arange(0, S, 256), np.arange(255, S, 256), rng.integers(0, S, 16)]))
    for h in (0, 2, 4):
        sl = lambda n: inputs.stored_values(x[n][:, h:h + 1])
        ro, rl = oracle.attention(sl("q"), sl("k"), sl("v"), 0.088, causal=causal, rows=rows)
        assert_bf16_parity(o[:, h:h + 1, rows], lse[:, h:h + 1, rows], ro, rl, f"H=5 S={S} causal={causal} h={h}")


# ------------------------------------------------------------------ running-max raises

def test_bf16_running_max_rises_across_tiles(ta, dev, dense_waves):
    # one query/key dimension carries a score ramp along the key index (about
    # 9 base-2 units per 64 keys), so the running max is raised again and
    # again after the first tile and the accumulator rescale runs; a rescale
    # left out or applied twice would weight early keys by a factor 2^9 off
    B, H, S, D = 1, 2, 1000, 128
    x = inputs.mha_inputs(B, H, S, S, D, seed=41)
    q = inputs.stored_values(x["q"]).copy()
    k = inputs.stored_values(x["k"]).copy()
    scale = float(np.float32(D ** -0.5))
    q[..., 0] = 1.0
    ramp = (9.0 / 64.0) * np.log(2.0) / scale  # natural-log score units per key
    k[..., 0] = (ramp * np.arange(S, dtype=np.float64)).astype(np.float32)
    y = dict(x, q=inputs.f32_to_bf16_bits(q), k=inputs.f32_to_bf16_bits(k))
    for causal in (False, True):
        o, lse = _run_mha(ta, dev, y, causal, scale)
        ro, rl = oracle.attention(*_vals(y, "qkv"), scale, causal=causal)
        assert_bf16_parity(o, lse, ro, rl, f"score ramp causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("jump", [24.0, 200.0, -200.0])
def test_running_max_jumps_inside_the_sequence(ta, dev, jump, D, dense_waves):
    # from key 640 on, one query/key dimension adds `jump` base-2 units to
    # every score: exponentials taken against the running max of the keys
    # before would reach 2^24 or overflow to inf (or, for a drop, underflow
    # to 0), so the step has to detect it and take the exact tile max
    B, H, S = 1, 2, 1000
    x = inputs.mha_inputs(B, H, S, S, D, seed=44)
    q = inputs.stored_values(x["q"]).copy()
    k = inputs.stored_values(x["k"]).copy()
    scale = float(np.float32(D ** -0.5))
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[..., 640:, 0] = jump * np.log(2.0) / scale
    y = dict(x, q=inputs.f32_to_bf16_bits(q), k=inputs.f32_to_bf16_bits(k))
    for causal in (False, True):
        o, lse = _run_mha(ta, dev, y, causal, scale)
        ro, rl = oracle.attention(*_vals(y, "qkv"), scale, causal=causal)
        assert_bf16_parity(o, lse, ro, rl, f"score jump {jump} D={D} causal={causal}")


def test_grouped_heads_score_jump(ta, dev, dense_waves):
    # the grouped-KV path shares the dense kernel's overflow check and exact
    # recompute: a 200-unit jump in the keys of one KV head
    B, H, Hkv, S, D = 1, 4, 2, 700, 128
    x = inputs.mha_inputs(B, H, S, S, D, seed=45, Hkv=Hkv)
    q = inputs.stored_values(x["q"]).copy()
    k = inputs.stored_values(x["k"]).copy()
    scale = float(np.float32(D ** -0.5))
    q[..., 0] = 1.0
    k[..., 0] = 0.0
    k[:, 1, 400:, 0] = 200.0 * np.log(2.0) / scale
    y = dict(x, q=inputs.f32_to_bf16_bits(q), k=inputs.f32_to_bf16_bits(k))
    qd, kd, vd = (to_dev(y[n], dev) for n in "qkv")
    for causal in (False, True):
        o, lse = ta.attn_fwd_ex(qd, kd, vd, causal=causal, scale=scale)
        torch.cuda.synchronize()
        ro, rl = oracle.attention_masked(*_vals(y, "qkv"), scale, causal=causal)
        assert_bf16_parity(to_np(o), to_np(lse), ro, rl, f"grouped score jump causal={causal}")


@pytest.mark.parametrize("H", [32, 64, 128])
def test_mla_running_max_rises_across_tiles(ta, dev, H):
    # the rotary part carries a score ramp along each batch's keys (about 9
    # base-2 units per 128 keys) and is not part of the values, so O stays
    # small while the running max of every head rises tile after tile inside
    # the pieces (16384 keys per batch: several tiles per piece)
    lens = [16384, 16384, 9000, 16384]
    B = len(lens)
    m = inputs.mla_inputs(B, H, seed=42 + H, kv_len=1)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = int(indptr[-1])
    g = np.random.default_rng(43 + H)
    m["kv"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 512), dtype=np.float32) * np.float32(0.3))
    scale = float(np.float32(576 ** -0.5))
    u = np.full(64, 0.5, dtype=np.float32)
    qpe = np.broadcast_to(u, (B, H, 64)) + g.standard_normal((B, H, 64), dtype=np.float32) * np.float32(0.01)
    m["q_pe"] = inputs.f32_to_bf16_bits(qpe.astype(np.float32))
    per_key = (9.0 / 128.0) * np.log(2.0) / (scale * float(u @ u))
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.float64)
    m["k_pe"] = inputs.f32_to_bf16_bits((per_key * pos)[:, None].astype(np.float32) * u[None, :])
    m["indptr"] = indptr
    o, lse = _run_mla(ta, dev, m, scale)
    ro, rl = oracle.mla_decode(*_mla_vals(m), indptr, scale)
    assert_bf16_parity(o, lse, ro, rl, f"mla score ramp H={H}")


# ------------------------------------------------------------------ split count, workspace cap

def _ragged_mla(dev, lens, H, seed):
    m = inputs.mla_inputs(len(lens), H, seed=seed, kv_len=1)
    indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    n = max(int(indptr[-1]), 1)
    g = np.random.default_rng(seed + 1)
    m["kv"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 512), dtype=np.float32) * np.float32(0.3))
    m["k_pe"] = inputs.f32_to_bf16_bits(g.standard_normal((n, 64), dtype=np.float32) * np.float32(0.3))
    m["indptr"] = indptr
    return m


@pytest.mark.parametrize("H", [64, 128])
def test_mla_result_does_not_depend_on_the_split_count(ta, dev, H, monkeypatch):
    # TATTN_MLA_SPLITS replaces the compute-unit count as the number of split
    # workgroups: one workgroup for everything, a few, and more workgroups than
    # compute units all agree with the oracle and with the default split
    lens = [3000, 1, 777, 0, 4096, 65]
    m = _ragged_mla(dev, lens, H, 51 + H)
    scale = float(np.float32(576 ** -0.5))
    ro, rl = oracle.mla_decode(*_mla_vals(m), m["indptr"], scale)
    o0, l0 = _run_mla(ta, dev, m, scale)
    for splits in (1, 3, 7, 64, 300, 1000):
        monkeypatch.setenv("TATTN_MLA_SPLITS", str(splits))
        o, lse = _run_mla(ta, dev, m, scale)
        assert_bf16_parity(o, lse, ro, rl, f"mla H={H} splits={splits}")
        empty = np.array(lens) == 0
        assert np.abs(o - o0).max() <= 1e-2 and np.abs(lse[~empty] - l0[~empty]).max() <= 1e-3
        assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    monkeypatch.delenv("TATTN_MLA_SPLITS")


def test_mla_workspace_cap_reports_oom_and_writes_nothing(ta, dev, monkeypatch):
    # a cap below the workspace the call needs: TATTN_ERR_OOM before any
    # launch, outputs untouched
    from tiled_attention_12_amd._binding import TattnError, TATTN_ERR_OOM
    m = _ragged_mla(dev, [500, 20], 128, 61)
    args = [to_dev(m[n], dev) for n in ("q", "q_pe", "kv", "k_pe")]
    ind = to_dev(m["indptr"], dev)
    out = torch.full((2, 128, 512), 3.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((2, 128), 3.0, dtype=torch.float32, device=dev)
    monkeypatch.setenv("TATTN_WS_LIMIT_BYTES", "4096")
    with pytest.raises(TattnError) as err:
        ta.mla_decode(*args, ind, 0.05, out=out, lse=lse)
    assert err.value.status == TATTN_ERR_OOM
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0)) and bool(torch.all(lse == 3.0))
    monkeypatch.delenv("TATTN_WS_LIMIT_BYTES")
    o, l2 = ta.mla_decode(*args, ind, 0.05, out=out, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(*_mla_vals(m), m["indptr"], 0.05)
    assert_bf16_parity(to_np(o), to_np(l2), ro, rl, "mla after the capped call")


def test_explicit_stream_gives_the_default_stream_result(ta, dev):
    # a caller's own stream (same device) is used for the launch; the result
    # is bit-identical to the call on the current stream
    x = inputs.mha_inputs(1, 4, 300, 300, 128, seed=8800)
    q, k, v = (to_dev(x[n], dev) for n in "qkv")
    o0, l0 = ta.attn_fwd(q, k, v, causal=True)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    o1, l1 = ta.attn_fwd(q, k, v, causal=True, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("fn", ["mla_decode", "mla_decode_noalloc"])
@pytest.mark.parametrize("B,H", [(1, 7), (5, 128)])
def test_mla_no_keys_in_any_batch(ta, dev, fn, B, H):
    # every batch empty (N = 0): kv and k_pe are empty tensors (null pointers
    # at the C ABI); every row gets O = 0 and LSE = -inf
    rng = np.random.default_rng(8900 + B)
    q = to_dev(inputs.f32_to_bf16_bits(rng.standard_normal((B, H, 512), dtype=np.float32)), dev)
    qpe = to_dev(inputs.f32_to_bf16_bits(rng.standard_normal((B, H, 64), dtype=np.float32)), dev)
    kv = torch.empty((0, 512), dtype=torch.bfloat16, device=dev)
    kpe = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    indptr = torch.zeros(B + 1, dtype=torch.int32, device=dev)
    o = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=dev)
    getattr(ta, fn)(q, qpe, kv, kpe, indptr, 576 ** -0.5, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0).item() and torch.all(torch.isneginf(lse)).item()
