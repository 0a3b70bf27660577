"""The workloads the layer is checked and measured on.

Shapes follow the pages: 512 routed experts per layer, 10 active plus one always-on
shared expert, 48 layers [Strata 与 Qwen3.8-Flash-Next (telli.sh), section
稀疏架构创造了机会]; at most three draft tokens verified together with the real one
[same page, section 推测解码只有在验证通过时才节省计算]; expert weights at 4 bit, mixed
layers at 6 bit, a dense projection at 8 bit [本地部署Qwen3.8-Flash-Next模型的两条路线
(blog.cycleuser.org), section 精度和内存占用], and experts at 2-3 bit in the low-bit
tiers [Strata 与 Qwen3.8-Flash-Next (telli.sh)]; prefill lengths 8192 and 32768 are the
sizes of that page's prefill table (section 性能对比).
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # stable integer id, part of every seed
    d: int                   # d_model
    E: int                   # routed experts
    k: int                   # experts selected per token
    F: int                   # expert FFN width
    T: int                   # tokens per call
    routed_fmt: str = "int4_g32"
    shared_fmt: str = "int4_g32"
    router_fmt: str = "fp32"
    bias: str = "none"       # "none" | "zipf"
    layers: int = 1
    extra_T: tuple = field(default_factory=tuple)

    @property
    def pairs(self):
        return self.T * self.k


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_d256_e16_top2", 0, d=256, E=16, k=2, F=128, T=4),
        Workload("decode_d2048_e512_top10_t1", 1, d=2048, E=512, k=10, F=512, T=1),
        Workload("decode_sweep_48_layers", 2, d=2048, E=512, k=10, F=512, T=1,
                 bias="zipf", layers=48, extra_T=(4,)),
        Workload("prefill_8192_zipf", 3, d=2048, E=512, k=10, F=512, T=8192, bias="zipf"),
        Workload("prefill_32768_mixed", 4, d=2048, E=512, k=10, F=512, T=32768,
                 routed_fmt="int4_g32", shared_fmt="int6_g32", router_fmt="int8_row",
                 bias="zipf"),
        # parity cases only: every expert at 6 bit, at decode sizes, so that the few-token
        # kernels' int6 path is checked (the prefill workload reaches int6 only through the
        # grouped GEMM); the 8-bit router where its kernels have the width (d = 2048)
        Workload("int6_d2048_e64_top10", 5, d=2048, E=64, k=10, F=512, T=4,
                 routed_fmt="int6_g32", shared_fmt="int6_g32", router_fmt="int8_row"),
        Workload("int6_tiny_d256_e16_top2", 6, d=256, E=16, k=2, F=128, T=33,
                 routed_fmt="int6_g32", shared_fmt="int6_g32"),
        # lower-bit plain codecs for the experts (the pages' 2-3 bit expert tiers): the
        # decode shape with every expert (routed and shared) at 3 or 2 bits, and tiny
        # shapes for the grouped GEMM's decoders
        Workload("int3_d2048_e512_top10", 7, d=2048, E=512, k=10, F=512, T=1,
                 routed_fmt="int3_g32", shared_fmt="int3_g32"),
        Workload("int2_d2048_e512_top10", 8, d=2048, E=512, k=10, F=512, T=1,
                 routed_fmt="int2_g32", shared_fmt="int2_g32"),
        Workload("int3_tiny_d256_e16_top2", 9, d=256, E=16, k=2, F=128, T=33,
                 routed_fmt="int3_g32", shared_fmt="int3_g32"),
        Workload("int2_tiny_d256_e16_top2", 10, d=256, E=16, k=2, F=128, T=33,
                 routed_fmt="int2_g32", shared_fmt="int2_g32"),
    ]
}
