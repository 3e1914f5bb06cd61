"""Host-side checks of the C ABI (CPU only, nothing is launched).

* the library loads and exports every function include/dsv4_attn.h declares;
* every argument error is reported with its status code and a message before
  any device work (descriptors carry dummy device pointers that the host side
  must never dereference).
"""
import ctypes
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HEADER = os.path.join(ROOT, "include", "dsv4_attn.h")

from hybrid_sparse_mqa_amd import _native as N  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(N.LIB_PATH), reason="HIP library not built")

OK, INVALID, UNSUPPORTED = 0, 1, 2
FAKE = 0x7F0000000000  # never dereferenced by the host side


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsv4_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = N.load()
    names = declared_functions()
    assert "dsv4_attn_forward" in names and "dsv4_attn_gather_slots" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_abi_version():
    assert N.load().dsv4_abi_version() == 2


def desc(dtype, shape, stride=None, data=FAKE):
    d = N.Tensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride = [1] * len(shape)
        for i in range(len(shape) - 2, -1, -1):
            stride[i] = stride[i + 1] * shape[i + 1]
    for i, (s, st) in enumerate(zip(shape, stride)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def base_args(R=4, T=4, H=64, B=2, K=512, fp8=False):
    pool = desc(N.DSV4_U8, [8, 149504]) if fp8 else desc(N.DSV4_BF16, [8 * 256, 512])
    return dict(
        q=desc(N.DSV4_BF16, [T, H, 512]),
        swa_pool=pool,
        swa_page_table=desc(N.DSV4_I32, [B, 4]),
        extra_pool=pool if R else None,
        extra_page_table=desc(N.DSV4_I32, [B, 3]) if R else None,
        c4_indices=desc(N.DSV4_I32, [T, K]) if R == 4 else None,
        seq_lens=desc(N.DSV4_I32, [B]),
        qo_indptr=desc(N.DSV4_I32, [B + 1]),
        sink=desc(N.DSV4_F32, [H]),
        compress_ratio=R,
        window=128,
        scale=512 ** -0.5,
        out=desc(N.DSV4_BF16, [T, H, 512]),
        lse=desc(N.DSV4_F32, [T, H]),
    )


def call(**kw):
    L = N.load()
    keys = ["q", "swa_pool", "swa_page_table", "extra_pool", "extra_page_table", "c4_indices", "seq_lens",
            "qo_indptr", "sink"]
    args = [N.ref(kw[k]) for k in keys]
    rc = L.dsv4_attn_forward(*args, kw["compress_ratio"], kw["window"], kw["scale"], N.ref(kw["out"]),
                             N.ref(kw["lse"]), None)
    return rc, L.dsv4_last_error().decode()


def mutate(**changes):
    kw = base_args(**changes.pop("base", {}))
    kw.update(changes)
    return kw


CASES = [
    ("ratio 3", mutate(compress_ratio=3), UNSUPPORTED, "compress_ratio"),
    ("ratio 64", mutate(compress_ratio=64), UNSUPPORTED, "compress_ratio"),
    ("head_dim 576", mutate(q=desc(N.DSV4_BF16, [4, 64, 576])), INVALID, "q"),
    ("no heads", mutate(q=desc(N.DSV4_BF16, [4, 0, 512]), out=desc(N.DSV4_BF16, [4, 0, 512])), INVALID, "heads"),
    ("129 heads", mutate(base=dict(H=129)), INVALID, "heads"),
    ("window 0", mutate(window=0), INVALID, "window"),
    ("c4 missing", mutate(c4_indices=None), INVALID, "c4_indices"),
    ("extra pool missing", mutate(extra_pool=None), INVALID, "extra_pool"),
    ("extra table missing", mutate(extra_page_table=None), INVALID, "extra_page_table"),
    ("q dtype", mutate(q=desc(N.DSV4_F32, [4, 64, 512])), INVALID, "dtype"),
    ("q strided last dim", mutate(q=desc(N.DSV4_BF16, [4, 64, 512], [65536, 1024, 2])), INVALID, "contiguous"),
    ("q misaligned", mutate(q=desc(N.DSV4_BF16, [4, 64, 512], data=FAKE + 2)), INVALID, "aligned"),
    ("qo_indptr length", mutate(qo_indptr=desc(N.DSV4_I32, [2])), INVALID, "qo_indptr"),
    ("table batch", mutate(swa_page_table=desc(N.DSV4_I32, [3, 4])), INVALID, "swa_page_table"),
    ("c4 rows", mutate(c4_indices=desc(N.DSV4_I32, [5, 512])), INVALID, "c4_indices"),
    ("sink heads", mutate(sink=desc(N.DSV4_F32, [63])), INVALID, "sink"),
    ("out shape", mutate(out=desc(N.DSV4_BF16, [4, 64, 448])), INVALID, "out"),
    ("lse dtype", mutate(lse=desc(N.DSV4_BF16, [4, 64])), INVALID, "lse"),
    ("pool width", mutate(swa_pool=desc(N.DSV4_BF16, [2048, 576])), INVALID, "swa_pool"),
    ("pool dtype", mutate(swa_pool=desc(N.DSV4_F32, [2048, 512])), INVALID, "swa_pool"),
    ("fp8 page bytes", mutate(swa_pool=desc(N.DSV4_U8, [8, 149000])), INVALID, "swa_pool"),
    ("mixed formats", mutate(extra_pool=desc(N.DSV4_U8, [8, 149504])), UNSUPPORTED, "same KV format"),
    ("seq_lens dtype", mutate(seq_lens=desc(N.DSV4_F32, [2])), INVALID, "seq_lens"),
    ("null q data", mutate(q=desc(N.DSV4_BF16, [4, 64, 512], data=0)), INVALID, "NULL"),
    ("scale nan", mutate(scale=float("nan")), INVALID, "scale"),
]


@pytest.mark.parametrize("name,kw,code,msg", CASES, ids=[c[0] for c in CASES])
def test_forward_argument_errors(name, kw, code, msg):
    rc, err = call(**kw)
    assert rc == code, (rc, err)
    assert msg.lower() in err.lower(), err


def test_ratio_zero_ignores_extra_arguments_and_empty_batch_is_ok():
    kw = base_args(R=0, T=0)
    rc, err = call(**kw)
    assert rc == OK, err


def test_gather_slots_argument_errors():
    L = N.load()
    kw = base_args(R=128)
    small = desc(N.DSV4_I32, [4, 128 + 767])  # needs window + 256 * 3 = 896
    counts = desc(N.DSV4_I32, [4, 2])
    rc = L.dsv4_attn_gather_slots(N.ref(kw["swa_page_table"]), N.ref(kw["extra_page_table"]), None,
                                  N.ref(kw["seq_lens"]), N.ref(kw["qo_indptr"]), 4, 128, 128, N.ref(small),
                                  N.ref(counts), None)
    assert rc == INVALID and "width" in L.dsv4_last_error().decode()
    rc = L.dsv4_attn_gather_slots(N.ref(kw["swa_page_table"]), N.ref(kw["extra_page_table"]), None,
                                  N.ref(kw["seq_lens"]), N.ref(kw["qo_indptr"]), 4, 5, 128, N.ref(small),
                                  N.ref(counts), None)
    assert rc == UNSUPPORTED


def test_kv_pack_argument_errors():
    L = N.load()
    k = desc(N.DSV4_BF16, [4, 512])
    slots = desc(N.DSV4_I32, [4])
    pool = desc(N.DSV4_U8, [2, 149504])

    def call(k_, s_, p_):
        return L.dsv4_kv_pack_fp8(N.ref(k_), N.ref(s_), N.ref(p_), None)

    assert call(desc(N.DSV4_F32, [4, 512]), slots, pool) == INVALID
    assert call(desc(N.DSV4_BF16, [4, 448]), slots, pool) == INVALID
    assert call(k, desc(N.DSV4_I32, [3]), pool) == INVALID
    assert call(k, slots, desc(N.DSV4_BF16, [512, 512])) == UNSUPPORTED
    assert "packed FP8" in L.dsv4_last_error().decode()
    assert call(desc(N.DSV4_BF16, [4, 512], stride=[516, 1]), slots, pool) == INVALID  # rows not 16-byte aligned
    assert call(k, slots, desc(N.DSV4_U8, [2, 149504], stride=[150000, 1])) == INVALID
    # no rows: nothing to launch
    assert call(desc(N.DSV4_BF16, [0, 512]), desc(N.DSV4_I32, [0]), pool) == 0


def test_c4_topk_argument_errors():
    L = N.load()

    def call(s_, n_, i_):
        return L.dsv4_c4_topk(N.ref(s_), N.ref(n_), N.ref(i_), None)

    sc, nc = desc(N.DSV4_F32, [4, 1000]), desc(N.DSV4_I32, [4])
    assert call(sc, nc, desc(N.DSV4_I32, [4, 0])) == UNSUPPORTED
    assert call(sc, nc, desc(N.DSV4_I32, [4, 4096])) == UNSUPPORTED
    assert call(desc(N.DSV4_BF16, [4, 1000]), nc, desc(N.DSV4_I32, [4, 512])) == INVALID
    assert call(sc, desc(N.DSV4_I32, [3]), desc(N.DSV4_I32, [4, 512])) == INVALID
    assert call(sc, nc, desc(N.DSV4_I32, [5, 512])) == INVALID
    assert call(desc(N.DSV4_F32, [0, 1000]), desc(N.DSV4_I32, [0]), desc(N.DSV4_I32, [0, 512])) == 0


def test_read_probe_argument_errors():
    L = N.load()

    def call(buf, nbytes, wgs, sink):
        return L.dsv4_read_probe(ctypes.c_void_p(buf), nbytes, wgs, ctypes.c_void_p(sink), None)

    assert call(FAKE, 1000, 256, FAKE) == INVALID  # not a multiple of 16
    assert call(FAKE, -16, 256, FAKE) == INVALID
    assert call(FAKE, 1 << 20, 0, FAKE) == INVALID
    assert call(FAKE, 1 << 20, (1 << 20) + 1, FAKE) == INVALID
    assert call(None, 1 << 20, 256, FAKE) == INVALID
    assert call(FAKE + 8, 1 << 20, 256, FAKE) == INVALID
    assert call(FAKE, 1 << 20, 256, None) == INVALID
    assert call(FAKE, 1 << 20, 256, FAKE + 4) == INVALID
    assert call(None, 0, 256, None) == OK  # nothing to read: nothing launched


def test_plan_is_host_only_and_sane():
    L = N.load()
    s = ctypes.c_int32()
    c = ctypes.c_int32()
    assert L.dsv4_attn_plan(64, 64, 128, 128, 0, 4, 0, ctypes.byref(s), ctypes.byref(c), None) == 0
    assert c.value % 32 == 0 and s.value * c.value >= 128 + 1024
    for fp8 in (0, 1):
        assert L.dsv4_attn_plan(32, 64, 4, 128, 512, 8, fp8, ctypes.byref(s), ctypes.byref(c), None) == 0
        assert s.value * c.value >= 640 and (s.value - 1) * c.value < 640
        assert c.value >= (32 if fp8 else 128)
    assert L.dsv4_attn_plan(32, 64, 7, 128, 512, 8, 0, ctypes.byref(s), ctypes.byref(c), None) == UNSUPPORTED
    assert L.dsv4_attn_set_split_keys(33) == INVALID
    assert L.dsv4_attn_set_split_keys(2064) == INVALID
    assert L.dsv4_attn_set_split_keys(64) == 0
    assert L.dsv4_attn_plan(32, 64, 4, 128, 512, 8, 0, ctypes.byref(s), ctypes.byref(c), None) == 0
    assert c.value == 64 and s.value == 10
    assert L.dsv4_attn_set_split_keys(0) == 0
    k = ctypes.c_int32()
    # bf16 with more than 16 heads: the 32-head role kernel, splitting keys to fill the chip
    assert L.dsv4_attn_plan(32, 64, 4, 128, 512, 8, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 3 and s.value == 4  # (without a GPU the plan assumes 256 compute units)
    # 16 heads or fewer: the 16-head kernel
    assert L.dsv4_attn_plan(32, 16, 4, 128, 512, 8, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 1
    # 128 rows x two 32-head blocks fill the chip without splitting keys: the role kernel, one split
    assert L.dsv4_attn_plan(128, 64, 4, 128, 512, 64, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 3 and s.value == 1
    # 64 rows x two 32-head blocks fill the chip with two splits: the role kernel
    assert L.dsv4_attn_plan(64, 64, 128, 128, 0, 4, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 3 and s.value == 2
    # 128 rows of 1152 keys: the role kernel's grid (128 x 2 x 2) would need two rounds: the 64-head
    # kernel, in two equal splits (not 1024 + 128)
    assert L.dsv4_attn_plan(128, 64, 128, 128, 0, 4, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 4 and s.value == 2 and c.value == 576
    # C4 decode: 256 rows (512 role workgroups, two rounds) the 64-head kernel; 192 rows (1.5 rounds)
    # and 128 rows (one) the role kernel
    assert L.dsv4_attn_plan(256, 64, 4, 128, 512, 32, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 4 and s.value == 1
    assert L.dsv4_attn_plan(192, 64, 4, 128, 512, 32, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 3 and s.value == 1
    assert L.dsv4_attn_plan(128, 64, 4, 128, 512, 32, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 3 and s.value == 1
    # packed FP8, 8 rows: the 32-head grid (8 x 2 x 10 splits) fits 256 compute units once
    assert L.dsv4_attn_plan(8, 64, 4, 128, 512, 1024, 1, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 6 and 8 * 2 * s.value <= 256
    # packed FP8, 256 rows: the 64-head kernel
    assert L.dsv4_attn_plan(256, 64, 4, 128, 512, 1024, 1, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 5
    # packed FP8, 32 rows: the 32-head grid fits once with 5 tiles per split; 64 rows: 10 tiles, the 64-head kernel
    assert L.dsv4_attn_plan(32, 64, 4, 128, 512, 1024, 1, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 6 and c.value <= 192
    assert L.dsv4_attn_plan(64, 64, 4, 128, 512, 1024, 1, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 5
    # packed FP8 with at most 32 heads: always the 32-head kernel
    assert L.dsv4_attn_plan(256, 32, 4, 128, 512, 1024, 1, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
    assert k.value == 6
    for forced in (1, 2, 3, 4):
        assert L.dsv4_attn_set_kernel(forced) == 0
        assert L.dsv4_attn_plan(64, 64, 128, 128, 0, 4, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
        assert k.value == forced
        assert L.dsv4_attn_plan(256, 64, 4, 128, 512, 1024, 1, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
        assert k.value == 5  # FP8 pools ignore a forced bf16 variant
    for forced in (5, 6):
        assert L.dsv4_attn_set_kernel(forced) == 0
        assert L.dsv4_attn_plan(8, 64, 4, 128, 512, 1024, 1, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
        assert k.value == forced
        assert L.dsv4_attn_plan(64, 64, 128, 128, 0, 4, 0, ctypes.byref(s), ctypes.byref(c), ctypes.byref(k)) == 0
        assert k.value == 3  # bf16 pools ignore a forced FP8 variant
    for bad in (7, -1, 32):
        assert L.dsv4_attn_set_kernel(bad) == INVALID
    assert L.dsv4_attn_set_kernel(0) == 0
