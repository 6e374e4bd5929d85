"""The Python binding's argument checks, on the CPU.

The C ABI receives bare pointers, so a tensor of the wrong size, dtype or layout would turn
into an out-of-bounds device access.  The binding checks every tensor argument against the
shapes the call implies before it calls the library.  Here the tensors are stand-ins that
carry only the attributes the checks read, and the library is replaced by a recorder: a
bad argument must raise ValueError with no library call, and a good call must reach the
library with the right sizes.
"""
import pytest

torch = pytest.importorskip("torch")

from bit_w4a4_quantized_amd import binding  # noqa: E402

U8, F16, F32, I8 = torch.uint8, torch.float16, torch.float32, torch.int8


class Dev:
    """A stand-in for a device tensor: shape, dtype, contiguity and a fake data pointer."""

    def __init__(self, shape, dtype, contiguous=True, cuda=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        self._contig = contiguous
        self.is_cuda = cuda
        self.device = torch.device("cuda:0")

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        return 4096

    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n

    def element_size(self):
        return torch.empty((), dtype=self.dtype).element_size()


class Recorder:
    """Records every C call and returns SVDQ_OK; size queries answer like the library."""

    def __init__(self, real):
        self.real = real
        self.calls = []

    def __getattr__(self, name):
        if name.endswith("_bytes"):
            return getattr(self.real, name)
        def fn(*args):
            self.calls.append((name, args))
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = Recorder(binding.lib())
    monkeypatch.setattr(binding, "lib", lambda: r)
    return r


FMT = "int4_e2m3"
M, K, N, R = 64, 256, 128, 32


def kb_args(**over):
    a = dict(xq=Dev(binding.code_shape(M, K, FMT), U8), xs=Dev(binding.scale_shape(M, K, FMT), F16),
             t=Dev((M, R), F16), wq=Dev(binding.code_shape(N, K, FMT), U8), ws=Dev(binding.scale_shape(N, K, FMT), F16),
             l2=Dev((R, N), F16), bias=Dev((N,), F16), y=Dev((M, N), F16))
    a.update(over)
    return a


def call_kb(a):
    return binding.svdq_gemm_w4a4_up(a["xq"], a["xs"], a["t"], a["wq"], a["ws"], a["l2"], a["bias"], K, FMT,
                                     y=a["y"], stream=0)


def test_kernel_b_good_call_reaches_the_library(rec):
    call_kb(kb_args())
    (name, args), = rec.calls
    assert name == "svdq_gemm_w4a4_up"
    assert args[7:12] == (M, N, K, R, binding.FORMATS[FMT])


@pytest.mark.parametrize("bad", [
    dict(l2=Dev((16, N), F16)),                  # branch rank of l2 differs from T's
    dict(t=Dev((M, 16), F16)),
    dict(y=Dev((M - 1, N), F16)),                # output smaller than [M, N]
    dict(y=Dev((M, N), F32)),
    dict(bias=Dev((N,), F32)),                   # fp32 bias
    dict(bias=Dev((N - 16,), F16)),              # short bias
    dict(xs=Dev(binding.scale_shape(M, K, FMT), F16, contiguous=False)),
    dict(xs=Dev(binding.scale_shape(M, K - 64, FMT), F16)),
    dict(wq=Dev(binding.code_shape(N, K - 64, FMT), U8)),   # codes of another K
    dict(ws=Dev(binding.scale_shape(N - 16, K, FMT), F16)),
    dict(xq=Dev(binding.code_shape(M, K, FMT), F16)),
    dict(xq=Dev(binding.code_shape(M, K, FMT), U8, cuda=False)),
    dict(l2=None),                               # T without a branch
    dict(t=None),                                # a branch without T
])
def test_kernel_b_rejects_bad_tensors(rec, bad):
    with pytest.raises(ValueError):
        call_kb(kb_args(**bad))
    assert rec.calls == []


def test_kernel_b_gelu_epilogue_checks_lambda(rec):
    a = kb_args()
    for lam in (Dev((N - 8,), F32), Dev((N,), F16), None):
        with pytest.raises(ValueError):
            binding.svdq_gemm_w4a4_up_gelu_smooth(a["xq"], a["xs"], a["t"], a["wq"], a["ws"], a["l2"], a["bias"],
                                                  lam, K, FMT, y=a["y"], stream=0)
    assert rec.calls == []


@pytest.mark.parametrize("bad", [
    dict(x_hat=Dev((M, K), F16, contiguous=False)),
    dict(x_hat=Dev((M, K), F32)),
    dict(l1t=Dev((R, K - 64), F16)),
    dict(xq=Dev(binding.code_shape(M + 1, K, FMT), U8)),
    dict(xs=Dev(binding.scale_shape(M, K, FMT), U8)),
    dict(t=Dev((M, R + 16), F16)),
    dict(l1t=None, t=Dev((M, R), F16)),          # T buffer without a branch
])
def test_kernel_a_rejects_bad_tensors(rec, bad):
    a = dict(x_hat=Dev((M, K), F16), l1t=Dev((R, K), F16), xq=None, xs=None, t=None)
    a.update(bad)
    with pytest.raises(ValueError):
        binding.svdq_quantize_down(a["x_hat"], a["l1t"], FMT, xq=a["xq"], xs=a["xs"], t=a["t"], no_workspace=True,
                                   stream=0)
    with pytest.raises(ValueError):
        binding.svdq_quantize_down_smooth(a["x_hat"], Dev((K,), F32), a["l1t"], FMT, xq=a["xq"], xs=a["xs"], t=a["t"],
                                          no_workspace=True, stream=0)
    assert rec.calls == []


def test_kernel_a_smoothing_factors_checked(rec):
    for lam in (Dev((K - 1,), F32), Dev((K,), F16)):
        with pytest.raises(ValueError):
            binding.svdq_quantize_down_smooth(Dev((M, K), F16), lam, None, FMT, xq=Dev(binding.code_shape(M, K, FMT), U8),
                                              xs=Dev(binding.scale_shape(M, K, FMT), F16), no_workspace=True, stream=0)
    assert rec.calls == []


def layer_args(**over):
    a = dict(x=Dev((M, K), F16), l1t=Dev((R, K), F16), wq=Dev(binding.code_shape(N, K, FMT), U8),
             ws=Dev(binding.scale_shape(N, K, FMT), F16), l2=Dev((R, N), F16), bias=Dev((N,), F16),
             y=Dev((M, N), F16), workspace=Dev((1 << 20,), U8))
    a.update(over)
    return a


def test_layer_good_call_reaches_the_library(rec):
    a = layer_args()
    binding.svdq_linear(a["x"], a["l1t"], a["wq"], a["ws"], a["l2"], a["bias"], FMT, workspace=a["workspace"],
                        y=a["y"], stream=0)
    (name, args), = rec.calls
    assert name == "svdq_linear" and args[6:11] == (M, N, K, R, binding.FORMATS[FMT])


@pytest.mark.parametrize("bad", [
    dict(l2=None),                               # branch half given
    dict(l1t=None),
    dict(l2=Dev((16, N), F16)),                  # ranks of L1 and L2 differ
    dict(l1t=Dev((R, K + 64), F16)),
    dict(bias=Dev((N + 16,), F16)),
    dict(y=Dev((M, N + 16), F16)),
    dict(wq=Dev(binding.code_shape(N, K + 64, FMT), U8)),
    dict(ws=Dev(binding.scale_shape(N, K, FMT), F32)),
    dict(x=Dev((M, K), F16, contiguous=False)),
])
@pytest.mark.parametrize("entry", ["svdq_linear", "svdq_linear_unfused", "svdq_linear_folded"])
def test_layer_rejects_bad_tensors(rec, bad, entry):
    a = layer_args(**bad)
    with pytest.raises(ValueError):
        if entry == "svdq_linear_folded":
            binding.svdq_linear_folded(a["x"], None, a["l1t"], a["wq"], a["ws"], a["l2"], a["bias"], None, FMT,
                                       workspace=a["workspace"], y=a["y"], stream=0)
        else:
            getattr(binding, entry)(a["x"], a["l1t"], a["wq"], a["ws"], a["l2"], a["bias"], FMT,
                                    workspace=a["workspace"], y=a["y"], stream=0)
    assert rec.calls == []


def test_folded_layer_checks_both_factor_vectors(rec):
    a = layer_args()
    for lam_in, lam_next in ((Dev((K + 4,), F32), None), (None, Dev((N - 8,), F32)), (Dev((K,), F16), None)):
        with pytest.raises(ValueError):
            binding.svdq_linear_folded(a["x"], lam_in, a["l1t"], a["wq"], a["ws"], a["l2"], a["bias"], lam_next, FMT,
                                       workspace=a["workspace"], y=a["y"], stream=0)
    assert rec.calls == []


def test_w4a16_glue_and_weight_entry_points_check_tensors(rec):
    x = Dev((M, K), F16)
    wq, ws = Dev(binding.code_shape(N, K, "int4"), U8), Dev(binding.scale_shape(N, K, "int4"), F16)
    for bad in (dict(ws=Dev((N, K // 64 - 1), F16)), dict(bias=Dev((N,), F32)), dict(y=Dev((M, N - 16), F16))):
        a = dict(x=x, wq=wq, ws=ws, bias=None, y=None)
        a.update(bad)
        with pytest.raises(ValueError):
            binding.svdq_gemm_w4a16(a["x"], a["wq"], a["ws"], a["bias"], y=a["y"], stream=0)
    with pytest.raises(ValueError):
        binding.svdq_gelu_tanh_smooth(Dev((M, N), F16), Dev((N - 8,), F32), stream=0)
    with pytest.raises(ValueError):
        binding.svdq_gelu_tanh_smooth(Dev((M, N), F16), Dev((N,), F32), out=Dev((M, N - 8), F16), stream=0)
    with pytest.raises(ValueError):
        binding.svdq_quantize_weight(Dev((N, K), F32), FMT, wq=Dev(binding.code_shape(N, K - 64, FMT), U8), stream=0)
    with pytest.raises(ValueError):
        binding.svdq_pack_weight(Dev((N, K), I8), Dev((N, K // 64 + 1), F16), "int4", stream=0)
    with pytest.raises(ValueError):
        binding.svdq_pack_weight(Dev((N, K), I8), Dev((N, K // 64), F16), "int4",
                                 ws=Dev(binding.scale_shape(N, K, "int4"), F32), stream=0)
    assert rec.calls == []


def test_prepared_layer_checks_once_and_calls_svdq_linear(rec, monkeypatch):
    # the weight side is checked at construction; a call checks only its activations and output
    # and reaches svdq_linear with the layer's sizes and the kept workspace
    a = layer_args()
    for bad in (dict(l2=Dev((16, N), F16)), dict(bias=Dev((N - 16,), F16)), dict(ws=Dev((3, N), F16)),
                dict(l1t=None)):
        b = dict(a, **bad)
        with pytest.raises(ValueError):
            binding.SvdqLinear(b["wq"], b["ws"], b["l1t"], b["l2"], b["bias"], K, FMT)
    layer = binding.SvdqLinear(a["wq"], a["ws"], a["l1t"], a["l2"], a["bias"], K, FMT)
    ws = Dev((1 << 20,), U8)
    monkeypatch.setattr(layer, "_workspace", lambda M: ws)
    layer._ws_bytes = 1 << 20
    for bad in (dict(x=Dev((M, K + 64), F16)), dict(x=Dev((M, K), F32)), dict(x=Dev((M, K), F16, contiguous=False)),
                dict(y=Dev((M, N + 16), F16)), dict(y=Dev((M, N), F32))):
        b = dict(a, **bad)
        with pytest.raises(ValueError):
            layer(b["x"], b["y"], stream=0)
    assert rec.calls == []
    layer(a["x"], a["y"], stream=0)
    (name, args), = rec.calls
    assert name == "svdq_linear" and args[6:11] == (M, N, K, R, binding.FORMATS[FMT]) and args[12] == 1 << 20
