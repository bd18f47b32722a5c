"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Bars: rollback windows, conv_state and every untouched element bit-exact; outputs
within 1e-5 + 1e-5|r| (fp32) or 1 bf16 ulp of the oracle's correctly rounded value.
Each test prints the case it is about to run before touching the GPU.
"""

import numpy as np
import pytest

import gpu_harness as gh
import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_conv1d_verify_amd._lib as L

    L.load()   # fail loudly if the HIP library is missing


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("key", [0, 1, 2, 3, 4, "4b", "4s", "t16"])
def test_workload_full_size(key):
    wl = workloads.WORKLOADS[key]
    _say(key, wl)
    rep = gh.check_against_oracle(workloads.make_inputs(wl))
    _say("ok", key, rep)


def _sweep():
    c = workloads.custom
    cases = []
    for T in (1, 2, 3, 8, 9, 16, 17, 32):
        for layout in ("dense", "dedup"):
            cases.append(c(f"T{T}_{layout}", n_seq=3, d_inner=1032, qk_channels=512,
                           head_dim=128, T=T, layout=layout, accept_offsets=True,
                           permute_slots=True, pad_frac=0.25, extra_slots=2))
    for D in (2, 3):
        for layout in ("dense", "dedup"):
            cases.append(c(f"D{D}_{layout}", n_seq=4, d_inner=520, qk_channels=256,
                           head_dim=64, d_conv=D, T=5, layout=layout))
            cases.append(c(f"D{D}_{layout}_off", n_seq=4, d_inner=520, qk_channels=256,
                           head_dim=64, d_conv=D, T=5, layout=layout, accept_offsets=True,
                           permute_slots=True))
    for xd, sd in (("f32", "f32"), ("bf16", "f32")):
        for layout in ("dense", "dedup"):
            for T in (1, 4, 16):
                cases.append(c(f"{xd}_{sd}_{layout}_T{T}", n_seq=3, d_inner=520,
                               qk_channels=256, head_dim=128 if xd == "bf16" else 64, T=T,
                               x_dtype=xd, state_dtype=sd, layout=layout,
                               accept_offsets=(T > 1), permute_slots=True, pad_frac=0.3))
    for hd in (4, 8, 16, 32, 64, 256):
        cases.append(c(f"head{hd}", n_seq=2, d_inner=1536, qk_channels=1024, head_dim=hd, T=4,
                       layout="dedup"))
    for hd in (4, 8, 16, 32, 256):
        cases.append(c(f"f32_head{hd}", n_seq=2, d_inner=768, qk_channels=512, head_dim=hd,
                       T=3, x_dtype="f32", state_dtype="f32"))
    cases.append(c("qk0", n_seq=2, d_inner=1024, qk_channels=0, T=6, layout="dedup"))
    cases.append(c("qk_all", n_seq=2, d_inner=1024, qk_channels=1024, T=6, layout="dense"))
    cases.append(c("qk_partial_wave", n_seq=2, d_inner=1024, qk_channels=384, T=6,
                   layout="dedup"))
    cases.append(c("ragged_8", n_seq=3, d_inner=8, qk_channels=8, head_dim=8, T=3))
    cases.append(c("ragged_many_waves", n_seq=2, d_inner=512 * 3 + 40, qk_channels=1024,
                   head_dim=128, T=7, layout="dedup", bias=False))
    cases.append(c("strided_x_out", n_seq=3, d_inner=1000, qk_channels=512, head_dim=128,
                   T=4, x_tok_stride=1024, layout="dedup", accept_offsets=True,
                   permute_slots=True))
    cases.append(c("big_eps", n_seq=2, d_inner=512, qk_channels=512, T=2, l2_eps=10.0))
    cases.append(c("zero_eps", n_seq=2, d_inner=512, qk_channels=512, T=2, l2_eps=0.0))
    cases.append(c("dyadic_exact", n_seq=2, d_inner=1024, qk_channels=512, T=8,
                   layout="dedup", dist="dyadic"))
    return cases


SWEEP = _sweep()


@pytest.mark.parametrize("wl", SWEEP, ids=[w.name for w in SWEEP])
def test_sweep(wl):
    _say(wl)
    gh.check_against_oracle(workloads.make_inputs(wl))


def test_dense_and_dedup_agree_on_gpu():
    base = dict(n_seq=6, d_inner=2048, qk_channels=1024, head_dim=128, T=9,
                accept_offsets=True, permute_slots=True, pad_frac=0.2)
    wd = workloads.custom("agree", layout="dense", **base)
    ww = workloads.custom("agree", layout="dedup", **base)
    _say("dense vs dedup", base)
    rd = gh.run_gpu(workloads.make_inputs(wd))
    rw = gh.run_gpu(workloads.make_inputs(ww))
    assert np.array_equal(rd["out"], rw["out"])
    assert np.array_equal(rd["conv_state"], rw["conv_state"])
    inp = workloads.make_inputs(wd)
    for i in gh.active_rows(inp):
        s = inp.slot_idx[i]
        for t in range(wd.T):
            assert np.array_equal(rw["windows"][s, :, t:t + 3], rd["windows"][s, t])
        assert np.array_equal(rd["windows"][s, wd.T - 1], rd["conv_state"][s, :, 0:3])


def test_batched_equals_per_row_calls():
    wl = workloads.custom("rows", n_seq=5, d_inner=1024, qk_channels=512, head_dim=128, T=6,
                          layout="dedup", accept_offsets=True, permute_slots=True,
                          pad_frac=0.2, extra_slots=1)
    inp = workloads.make_inputs(wl)
    _say("batched vs rows", wl)
    whole = gh.run_gpu(inp)
    import causal_conv1d_verify_amd as cv

    p = gh.DeviceProblem(inp)
    for i in range(wl.n_seq):
        cv.conv_verify_update_dedup(p.x[i:i + 1], p.weight, p.bias, p.conv_state, p.out[i:i + 1],
                                    p.windows, qk_channels=wl.qk_channels,
                                    head_dim=wl.head_dim, l2_eps=wl.l2_eps,
                                    slot_idx=p.slot_idx[i:i + 1],
                                    num_accept_tokens=p.nat[i:i + 1])
    rows = p.results()
    for k in ("out", "windows", "conv_state"):
        assert np.array_equal(rows[k], whole[k]), k


def test_special_values_move_as_bits():
    for xd, sd in (("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")):
        wl = workloads.custom(f"bits_{xd}_{sd}", n_seq=2, d_inner=512,
                              qk_channels=256, head_dim=128 if xd == "bf16" else 64, T=3,
                              x_dtype=xd, state_dtype=sd, layout="dedup")
        inp = workloads.make_inputs(wl)
        sb16 = np.array([0x8000, 0x0001, 0x807F, 0x7FA1, 0xFFC3, 0x7F80, 0xFF80], np.uint16)
        sb32 = np.array([0x80000000, 0x00000001, 0x807FFFFF, 0x7FA00001, 0xFFC00003,
                         0x7F800000, 0xFF800000], np.uint32).view(np.float32)
        inp.x[0, :, 300:307] = sb16 if xd == "bf16" else sb32
        inp.conv_state[1, 300:307, 2] = sb16 if sd == "bf16" else sb32
        _say("special values", xd, sd)
        gh.check_against_oracle(inp)


def test_empty_and_all_padded_batches():
    import torch

    import causal_conv1d_verify_amd as cv

    wl = workloads.custom("pads", n_seq=4, d_inner=512, qk_channels=256, head_dim=128, T=3,
                          layout="dense", pad_frac=1.0, permute_slots=True)
    inp = workloads.make_inputs(wl)
    assert (inp.slot_idx < 0).all()
    _say("all padded")
    gh.check_against_oracle(inp)
    _say("empty batch")
    p = gh.DeviceProblem(inp)
    before = p.results()
    cv.conv_verify_update_dense(p.x[:0], p.weight, p.bias, p.conv_state, p.out[:0], p.windows,
                                qk_channels=256, head_dim=128)
    after = p.results()
    for k in before:
        assert np.array_equal(before[k], after[k])
    torch.cuda.synchronize()


def test_out_of_range_rows_are_skipped():
    wl = workloads.custom("range", n_seq=6, d_inner=512, qk_channels=256, head_dim=128, T=4,
                          layout="dedup", accept_offsets=True)
    inp = workloads.make_inputs(wl)
    inp.slot_idx = np.arange(6, dtype=np.int32)
    inp.slot_idx[1] = wl.n_slots          # slot past the pool
    inp.slot_idx[2] = -7                  # negative, not -1
    inp.num_accept_tokens[3] = wl.state_len - 2   # window would run past the row
    inp.num_accept_tokens[4] = -1
    _say("out-of-range rows")
    gpu = gh.run_gpu(inp)
    ref_inp = workloads.Inputs(**{**inp.__dict__})
    ref_inp.slot_idx = inp.slot_idx.copy()
    ref_inp.slot_idx[[1, 2, 3, 4]] = -1
    ref_inp.num_accept_tokens = inp.num_accept_tokens.copy()
    ref_inp.num_accept_tokens[[3, 4]] = 0
    ref = oracle.run_inputs(ref_inp)
    gh.compare(gpu, ref, wl, [0, 5])


def test_nondefault_stream_and_repeatability():
    import torch

    wl = workloads.custom("stream", n_seq=8, d_inner=2048, qk_channels=1024, head_dim=128, T=8,
                          layout="dedup", accept_offsets=True, permute_slots=True)
    inp = workloads.make_inputs(wl)
    s = torch.cuda.Stream()
    _say("side stream")
    gh.check_against_oracle(inp, stream=s)
    a = gh.run_gpu(inp, stream=s)
    b = gh.run_gpu(inp)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_rejected_call_writes_nothing():
    import causal_conv1d_verify_amd as cv

    wl = workloads.custom("reject", n_seq=2, d_inner=512, qk_channels=256, head_dim=128, T=3)
    p = gh.DeviceProblem(workloads.make_inputs(wl))
    before = p.results()
    _say("rejected call")
    with pytest.raises(cv.CvError) as e:
        cv.conv_verify_update_dense(p.x, p.weight, p.bias, p.conv_state, p.out, p.windows,
                                    qk_channels=256, head_dim=96)
    assert e.value.code == -22
    after = p.results()
    for k in before:
        assert np.array_equal(before[k], after[k])
