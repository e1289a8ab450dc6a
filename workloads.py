"""Seeded synthetic inputs shaped like the pages' LLM linear-layer workloads.

This module is shared by the GPU tests, the benchmark and the CPU oracle's
tests, and it holds no GEMM arithmetic: it only draws random numbers, rounds
them to the storage formats, and (for the FP8 inputs) quantises them with
torch's own float8_e4m3fn cast, which is the input recipe of the FP8
workload.  The oracle's quantiser in ``oracle/quant.py`` is written
independently from the format definition, and a CPU test checks that the two
give the same bits.

Workload shapes (sources cited by short name: "GEMM compute-cost page" is
kwkr.cn/news/191298, "DeepGEMM page" is zwxr.cn/news/240083):

* tiny    64 x 64 x 64 -- the small correctness size of the DeepGEMM page,
          section 3.1; bf16 U[-1, 1], fp32 output.
* square  4096^3 -- the large size of the same section; bf16 N(0, 1).
* ffn_up / ffn_down -- the 7B FFN pair of the GEMM compute-cost page,
          section 2.1: [2048, 4096] x [4096, 16384] (+bias, GeLU) and
          [2048, 16384] x [16384, 4096]; weights N(0, 0.02).
* thin    the LM head of section 7.2 of the same page: M in {1, 8, 32, 64}
          rows against a [4096, 128256] weight.
* fp8     4096 x 14336 x 4096 with 1x128 activation scales and 128x128
          weight scales (DeepGEMM page, section 2.4); A has 0.1% outliers
          scaled by 20.  fp8_ragged is the same with M = 4097, N = 14335.

Random streams: tensor ``t`` of a workload with master seed ``s`` draws from a
``torch.Generator`` on the target device seeded with ``s * 256 + t``.  The
same seed gives the same values on the same device type and torch version.
"""

from dataclasses import dataclass, field

import torch

FP8_GROUP = 128
E4M3_MAX = 448.0

# tensor indices inside one workload's seed space
T_A, T_B, T_BIAS, T_OUTLIER = 1, 2, 3, 4
T_W8_CODES, T_W8_SCALES = 6, 7
T_W4_CODES, T_W4_SCALES = 8, 9


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    a_dist: str = "normal"      # "normal" or "uniform" (U[-1, 1])
    a_sigma: float = 1.0
    b_sigma: float = 1.0
    bias_sigma: float = 0.0     # 0: no bias
    epilogue: int = 0           # 0 none, 1 bias, 2 bias + tanh-GeLU
    out_f32: bool = False
    fp8: bool = False
    notes: dict = field(default_factory=dict, compare=False, hash=False)


WORKLOADS = {
    "tiny": Workload("tiny", 64, 64, 64, seed=1, a_dist="uniform", out_f32=True),
    "square": Workload("square", 4096, 4096, 4096, seed=2),
    "ffn_up": Workload("ffn_up", 2048, 16384, 4096, seed=3, b_sigma=0.02,
                       bias_sigma=0.02, epilogue=2),
    "ffn_down": Workload("ffn_down", 2048, 4096, 16384, seed=3, b_sigma=0.02),
    "thin_m1": Workload("thin_m1", 1, 128256, 4096, seed=4, b_sigma=0.02),
    "thin_m8": Workload("thin_m8", 8, 128256, 4096, seed=4, b_sigma=0.02),
    "thin_m32": Workload("thin_m32", 32, 128256, 4096, seed=4, b_sigma=0.02),
    "thin_m64": Workload("thin_m64", 64, 128256, 4096, seed=4, b_sigma=0.02),
    "fp8": Workload("fp8", 4096, 14336, 4096, seed=5, b_sigma=0.02, fp8=True),
    "fp8_ragged": Workload("fp8_ragged", 4097, 14335, 4096, seed=6, b_sigma=0.02, fp8=True),
}


def generator(seed, tensor_index, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 256 + int(tensor_index))
    return g


def draw(shape, dist, sigma, seed, tensor_index, device="cpu"):
    """fp32 samples: N(0, sigma) or U[-1, 1]."""
    g = generator(seed, tensor_index, device)
    if dist == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * sigma
    if dist == "uniform":
        return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * 2.0 - 1.0
    raise ValueError(dist)


def bf16(shape, dist, sigma, seed, tensor_index, device="cpu"):
    """Samples rounded to bfloat16 (torch's cast rounds to nearest even)."""
    return draw(shape, dist, sigma, seed, tensor_index, device).to(torch.bfloat16)


def bf16_inputs(w: Workload, device="cpu", rows=None):
    """(A [M,K], B [K,N], bias [N] or None), all bf16 and contiguous.

    ``rows`` overrides M (the thin-M workloads share one X and take its first
    ``M`` rows, so M = 1, 8, 32, 64 see nested inputs).
    """
    M = w.M if rows is None else rows
    a_full = bf16((64 if w.name.startswith("thin") else M, w.K), w.a_dist, w.a_sigma,
                  w.seed, T_A, device)
    a = a_full[:M].contiguous()
    b = bf16((w.K, w.N), "normal", w.b_sigma, w.seed, T_B, device)
    bias = None
    if w.bias_sigma > 0:
        bias = bf16((w.N,), "normal", w.bias_sigma, w.seed, T_BIAS, device)
    return a, b, bias


def thin_x(w: Workload, M, device="cpu"):
    """The first M rows of a thin-M workload's X (the same draws bf16_inputs uses)."""
    return bf16((64, w.K), w.a_dist, w.a_sigma, w.seed, T_A, device)[:M].contiguous()


def ffn_hidden(M, N, seed, device="cpu"):
    """Stand-in for the down-projection input H in parity tests: N(0, 1) bf16."""
    return bf16((M, N), "normal", 1.0, seed, 5, device)


def _pad_to(x, dim, multiple):
    size = x.shape[dim]
    pad = (-size) % multiple
    if pad == 0:
        return x
    shape = list(x.shape)
    shape[dim] = pad
    return torch.cat([x, torch.zeros(shape, dtype=x.dtype, device=x.device)], dim=dim)


def quantise_a_1x128(x):
    """[M, K] fp32 -> (e4m3fn codes [M, K], fp32 scales [M, ceil(K/128)]).

    scale = amax / 448 over the in-range elements of each (row, 128-wide K
    group), 1 for an all-zero group; code = cast(clamp(x / scale)).
    """
    M, K = x.shape
    xp = _pad_to(x, 1, FP8_GROUP)
    G = xp.shape[1] // FP8_GROUP
    amax = xp.view(M, G, FP8_GROUP).abs().amax(dim=2)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / E4M3_MAX)
    scaled = xp.view(M, G, FP8_GROUP) / s.unsqueeze(2)
    q = scaled.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(M, G * FP8_GROUP)
    return q[:, :K].contiguous(), s.contiguous()


def quantise_b_128x128(x):
    """[K, N] fp32 -> (e4m3fn codes [K, N], fp32 scales [ceil(K/128), ceil(N/128)])."""
    K, N = x.shape
    xp = _pad_to(_pad_to(x, 0, FP8_GROUP), 1, FP8_GROUP)
    G, H = xp.shape[0] // FP8_GROUP, xp.shape[1] // FP8_GROUP
    blocks = xp.view(G, FP8_GROUP, H, FP8_GROUP)
    amax = blocks.abs().amax(dim=(1, 3))
    s = torch.where(amax == 0, torch.ones_like(amax), amax / E4M3_MAX)
    scaled = blocks / s.view(G, 1, H, 1)
    q = scaled.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(G * FP8_GROUP, H * FP8_GROUP)
    return q[:K, :N].contiguous(), s.contiguous()


def fp8_inputs(w: Workload, device="cpu", M=None, N=None, K=None):
    """(qA e4m3fn [M,K], sA fp32, qB e4m3fn [K,N], sB fp32) for an FP8 workload.

    A ~ N(0, 1) with each element independently an outlier with probability
    0.001, multiplied by 20; B ~ N(0, b_sigma).  Shapes default to the
    workload's and may be overridden for small parity cases.
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    a = draw((M, K), "normal", w.a_sigma, w.seed, T_A, device)
    u = draw((M, K), "uniform", 1.0, w.seed, T_OUTLIER, device)
    a = torch.where((u + 1.0) * 0.5 < 0.001, a * 20.0, a)
    b = draw((K, N), "normal", w.b_sigma, w.seed, T_B, device)
    qa, sa = quantise_a_1x128(a)
    qb, sb = quantise_b_128x128(b)
    return qa, sa, qb, sb


def fp8_sources_bf16(w: Workload, device="cpu", M=None, N=None, K=None):
    """(A bf16 [M,K], B bf16 [K,N]): the FP8 workload's unquantised operands
    (same draws and outliers as ``fp8_inputs``) rounded to bf16, the inputs
    of the GPU quantisers."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    a = draw((M, K), "normal", w.a_sigma, w.seed, T_A, device)
    u = draw((M, K), "uniform", 1.0, w.seed, T_OUTLIER, device)
    a = torch.where((u + 1.0) * 0.5 < 0.001, a * 20.0, a)
    b = draw((K, N), "normal", w.b_sigma, w.seed, T_B, device)
    return a.to(torch.bfloat16), b.to(torch.bfloat16)


def w8_weights(K, N, seed, device="cpu"):
    """Synthetic operands of a weight-only int8 LM head: int8 codes Q [K, N]
    and fp32 scales S [ceil(K/128), N].

    Drawn directly rather than quantised: codes follow N(0, 32) rounded and
    clipped to [-127, 127] (the shape of round-to-nearest codes of Gaussian
    weights under a per-group max scaling) and scales are 4.6e-4 * (1 + 0.2 u),
    u ~ U[-1, 1] (about the max of 128 draws of N(0, 0.02), over 127).
    """
    q = draw((K, N), "normal", 32.0, seed, T_W8_CODES, device).round().clamp(-127, 127)
    G = (K + 127) // 128
    u = draw((G, N), "uniform", 1.0, seed, T_W8_SCALES, device)
    return q.to(torch.int8), (4.6e-4 * (1.0 + 0.2 * u)).to(torch.float32).contiguous()


def w4_weights(K, N, seed, device="cpu"):
    """Synthetic operands of a weight-only int4 LM head: packed bytes
    [K/2, N] (byte (r, n) = code (2r, n) in bits 0-3, code (2r+1, n) in bits
    4-7, two's complement) and fp32 scales S [ceil(K/128), N].

    Codes follow N(0, 2.4) rounded and clipped to [-7, 7] (round-to-nearest
    codes of Gaussian weights under a per-group max scaling: 7 * sigma / amax
    with amax about 2.9 sigma over 128 draws); scales are 8.3e-3 * (1 + 0.2 u),
    u ~ U[-1, 1] (about the max of 128 draws of N(0, 0.02), over 7).
    """
    if K % 2:
        raise ValueError("K must be even")
    q = draw((K, N), "normal", 2.4, seed, T_W4_CODES, device).round().clamp(-7, 7).to(torch.int16)
    nib = (q & 0x0F).to(torch.uint8)
    packed = (nib[0::2] | (nib[1::2] << 4)).contiguous()
    G = (K + 127) // 128
    u = draw((G, N), "uniform", 1.0, seed, T_W4_SCALES, device)
    return packed, (8.3e-3 * (1.0 + 0.2 * u)).to(torch.float32).contiguous()


def bits_u16(t):
    """bf16 tensor -> numpy uint16 codes (on CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def bits_u8(t):
    """float8 tensor -> numpy uint8 codes (on CPU)."""
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()
