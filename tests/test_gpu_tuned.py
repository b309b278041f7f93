"""Tuned configurations on the GPU: a tuned file overrides the table for its
exact shapes (queries report it, results stay within the parity bar), and the
tuner writes a file the library accepts."""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gemm_epilogues_mlp_amd import tune as T
from gpu_util import Run, assert_parity, dev, host, log

pytestmark = pytest.mark.gpu

M, N, K = 300, 264, 200


def _ids():
    def first_other(variant, avoid):
        return next(i for i in range(sw.swiglu_config_count())
                    if sw.swiglu_config_info(i)["variant"] == variant and i != avoid
                    and sw.swiglu_config_info(i)["family"] == 0)
    h = sw.swiglu_create(0)
    try:
        bi = sw.swiglu_query(h, M, N, K, sw.LAYOUT_INTERLEAVED)[1]["id"]
        bs = sw.swiglu_query(h, M, N, K, sw.LAYOUT_SEPARATE)[1]["id"]
        bg = sw.swiglu_query_unfused(h, M, N, K)["id"]
    finally:
        sw.swiglu_destroy(h)
    return (first_other(sw.VARIANT_INTERLEAVE, bi), first_other(sw.VARIANT_SYNC, bs),
            first_other(sw.VARIANT_GEMM, bg))


def test_tuned_file_overrides_the_table(tmp_path):
    ti, ts, tg = _ids()
    path = tmp_path / "tuned.txt"
    path.write_text(f"swiglu-tuned {sw.swiglu_config_signature():016x} gfx950\n"
                    f"2 {M} {N} {K} {ti}\n1 {M} {N} {K} {ts}\n3 {M} {N} {K} {tg}\n")
    log(f"tuned ids {ti} {ts} {tg}")
    h = sw.swiglu_create_tuned(0, str(path))
    try:
        assert sw.swiglu_query(h, M, N, K, sw.LAYOUT_INTERLEAVED)[1]["id"] == ti
        assert sw.swiglu_query(h, M, N, K, sw.LAYOUT_SEPARATE)[1]["id"] == ts
        assert sw.swiglu_query_unfused(h, M, N, K)["id"] == tg
        # other shapes keep the built-in table
        plain = sw.swiglu_create(0)
        try:
            for m, n, k in [(M + 8, N, K), (M, N, K + 8)]:
                assert sw.swiglu_query(h, m, n, k, sw.LAYOUT_INTERLEAVED)[1] == \
                    sw.swiglu_query(plain, m, n, k, sw.LAYOUT_INTERLEAVED)[1]
        finally:
            sw.swiglu_destroy(plain)
        rng = np.random.default_rng(5)
        a = I.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
        w1 = I.f32_to_bf16_bits(rng.standard_normal((K, N), dtype=np.float32) / np.sqrt(K))
        w2 = I.f32_to_bf16_bits(rng.standard_normal((K, N), dtype=np.float32) / np.sqrt(K))
        y_ref = oracle.swiglu_rows(a, w1, w2)
        t = __import__("torch")
        for layout, W1, W2 in [(sw.LAYOUT_INTERLEAVED, I.interleave_columns(w1, w2), None),
                               (sw.LAYOUT_SEPARATE, w1, w2)]:
            y = t.full((M, N), -1, dtype=t.int16, device="cuda")
            sw.swiglu_forward(h, dev(a), dev(W1), None if W2 is None else dev(W2), y, M, N, K,
                              layout)
            t.cuda.synchronize()
            assert_parity(host(y), y_ref, f"tuned forward, layout {layout}")
        # the unfused path (tuned GEMM config): its G and U against the oracle
        _, gu, uu = Run(h).unfused(dev(a), dev(w1), dev(w2), M, N, K)
        g_ref, u_ref = oracle.swiglu_rows(a, w1, w2, with_gate_up=True)[1:]
        assert_parity(host(gu), g_ref, "tuned unfused G")
        assert_parity(host(uu), u_ref, "tuned unfused U")
    finally:
        sw.swiglu_destroy(h)


def test_stale_file_is_refused_on_creation(tmp_path):
    path = tmp_path / "stale.txt"
    path.write_text("swiglu-tuned 0123456789abcdef gfx950\n")
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_create_tuned(0, str(path))
    assert e.value.status == sw.ERR_UNSUPPORTED


def test_tuner_writes_a_valid_file(tmp_path):
    out = tmp_path / "t.txt"
    msgs = []
    T.tune([(M, K, N)], variants=("interleave", "gemm"), out=str(out), reps=3,
           configs=[1, 2, 3, 15, 16, 17], margin=0.0, log=msgs.append)
    log("\n".join(msgs))
    assert len(msgs) == 2
    n = sw.swiglu_tuned_check(str(out))
    h = sw.swiglu_create_tuned(0, str(out))
    sw.swiglu_destroy(h)
    assert n <= 2


def test_tuner_covers_the_fp8_families(tmp_path):
    """The tuner times the FP8 (both orders) and MXFP8 configurations and its
    file is accepted; an FP8 entry it writes (or one written by hand) steers
    swiglu_forward_fp8 / _mx with config_id < 0, with results within the bar."""
    Mf, Kf, Nf = 192, 256, 264
    out = tmp_path / "t8.txt"
    msgs = []
    T.tune([(Mf, Kf, Nf)], variants=("fp8", "fp8-sync", "mxfp8"), out=str(out), reps=3,
           margin=0.0, log=msgs.append)
    log("\n".join(msgs))
    assert len(msgs) == 3
    sw.swiglu_tuned_check(str(out))
    # a hand-written entry for each family: the first configuration that is
    # not the table's choice
    h = sw.swiglu_create(0)
    try:
        picks = {}
        for v, order in [(sw.VARIANT_FP8, sw.VARIANT_INTERLEAVE), (sw.VARIANT_FP8_SYNC, sw.VARIANT_SYNC),
                         (sw.VARIANT_MXFP8, sw.VARIANT_MXFP8)]:
            builtin = sw.swiglu_query_fp8(h, Mf, Nf, Kf, order)["id"]
            picks[v] = next(i for i in range(sw.swiglu_config_count())
                            if sw.swiglu_config_info(i)["variant"] == v and i != builtin
                            and sw.swiglu_config_info(i)["family"] == 0)
    finally:
        sw.swiglu_destroy(h)
    path = tmp_path / "hand8.txt"
    path.write_text(f"swiglu-tuned {sw.swiglu_config_signature():016x} gfx950\n" +
                    "".join(f"{v} {Mf} {Nf} {Kf} {c}\n" for v, c in picks.items()))
    h = sw.swiglu_create_tuned(0, str(path))
    try:
        assert sw.swiglu_query_fp8(h, Mf, Nf, Kf, sw.VARIANT_AUTO)["id"] == picks[sw.VARIANT_FP8]
        assert sw.swiglu_query_fp8(h, Mf, Nf, Kf, sw.VARIANT_SYNC)["id"] == \
            picks[sw.VARIANT_FP8_SYNC]
        assert sw.swiglu_query_fp8(h, Mf, Nf, Kf, sw.VARIANT_MXFP8)["id"] == \
            picks[sw.VARIANT_MXFP8]
        t = __import__("torch")
        a, w1, w2 = I.make_inputs(Mf, Kf, Nf, 31)
        qa, sa = oracle.quantize_mx(I.bf16_bits_to_f32(a))
        qw, sW = oracle.quantize_mx(I.bf16_bits_to_f32(oracle.pack_kmajor_bf16(w1, w2)))
        d8 = lambda x: t.from_numpy(np.ascontiguousarray(x)).cuda()
        y = t.full((Mf, Nf), -1, dtype=t.int16, device="cuda")
        sw.swiglu_forward_mx(h, d8(qa), d8(sa), d8(qw), d8(sW), y, Mf, Nf, Kf, sa.shape[1])
        t.cuda.synchronize()
        assert_parity(host(y), oracle.swiglu_mx_rows(qa, sa, qw, sW), "tuned MXFP8 forward")
        # per-tensor FP8 (scale = max|x| / 448 per tensor), both orders
        xs = [I.bf16_bits_to_f32(x) for x in (a, w1, w2)]
        sc = [float(np.float32(np.max(np.abs(x)) / np.float32(448.0))) for x in xs]
        a8, w18, w28 = (oracle.quantize_e4m3(x, np.float32(1.0) / np.float32(c))
                        for x, c in zip(xs, sc))
        ref = oracle.swiglu_fp8_rows(a8, w18, w28, *sc)
        for order in (sw.VARIANT_AUTO, sw.VARIANT_SYNC):
            y.fill_(-1)
            sw.swiglu_forward_fp8(h, d8(a8), d8(oracle.pack_fp8_kmajor(w18, w28)), y, Mf, Nf, Kf,
                                  *sc, variant=order)
            t.cuda.synchronize()
            assert_parity(host(y), ref, f"tuned FP8 forward, order {order}")
    finally:
        sw.swiglu_destroy(h)
