"""The five workloads of the fused operators, named by what they are.

Shapes, distributions and tile sizes only; seeds and draw order live in
``inputs``.  Every workload models one GPU's share of a P-way tensor-parallel
(or model-parallel) job with the P logical shards' receive windows in local
HBM.
"""

from dataclasses import dataclass, field

F32 = 0
BF16 = 1


@dataclass(frozen=True)
class GemmRS:
    name: str
    P: int
    M: int          # rows of each A_p (= rows of the reduced output)
    N: int
    K: int
    in_dt: int
    slot_dt: int
    out_dt: int
    tile_m: int
    tile_n: int
    dist_a: tuple = ("normal", 1.0)
    dist_w: tuple = ("normal", 0.02)

    @property
    def flops(self):
        return 2.0 * self.P * self.M * self.N * self.K


@dataclass(frozen=True)
class GemvAR:
    name: str
    P: int
    Mb: int
    N: int
    K: int
    in_dt: int
    slot_dt: int
    out_dt: int
    tile_n: int

    @property
    def flops(self):
        return 2.0 * self.P * self.Mb * self.N * self.K


@dataclass(frozen=True)
class AgGemm:
    name: str
    P: int
    Mc: int
    N: int
    K: int
    tile_m: int
    tile_n: int

    @property
    def flops(self):
        return 2.0 * self.P * self.Mc * self.N * self.K


@dataclass(frozen=True)
class EmbbagA2A:
    name: str
    T: int
    R: int
    D: int
    B: int
    L: int
    P: int
    tile_bags: int
    alpha: float = 1.05


# GEMM+ReduceScatter, tiny: 4 shards of 256x256 fp32 U[-1,1), tile 64x64.
GEMM_RS_TINY = GemmRS("gemm_rs_tiny_p4_256_f32", P=4, M=256, N=256, K=256,
                      in_dt=F32, slot_dt=F32, out_dt=F32, tile_m=64, tile_n=64,
                      dist_a=("uniform",), dist_w=("uniform",))

# GEMV+AllReduce, decode: 8 shards, x_p 4x1024, W_p 1024x8192 bf16, fp32 partials.
GEMV_AR_DECODE = GemvAR("gemv_ar_decode_p8_4x1024x8192_bf16", P=8, Mb=4, N=8192, K=1024,
                        in_dt=BF16, slot_dt=F32, out_dt=BF16, tile_n=256)

# GEMM+ReduceScatter, row-parallel MLP-down: 8 shards of 8192x1792 . 1792x4096 bf16.
GEMM_RS_MLP = GemmRS("gemm_rs_mlpdown_p8_8192x4096x1792_bf16", P=8, M=8192, N=4096, K=1792,
                     in_dt=BF16, slot_dt=F32, out_dt=BF16, tile_m=256, tile_n=256)

# AllGather+GEMM, column-parallel: 8 chunks of 1024x4096, W 4096x1792 bf16.
AG_GEMM_COL = AgGemm("ag_gemm_colpar_p8_1024x4096x1792_bf16", P=8, Mc=1024, N=1792, K=4096,
                     tile_m=256, tile_n=256)

# Embedding-bag + All-to-All: 64 tables of 1e6 x 128 fp32, batch 16384, 20 per bag.
EMBBAG_DLRM = EmbbagA2A("embbag_a2a_t64_r1e6_d128_b16384_l20_p8", T=64, R=1_000_000, D=128,
                        B=16384, L=20, P=8, tile_bags=64)

# GEMM+AllReduce at the same row-parallel MLP-down shape: the ReduceScatter's
# folded chunks are gathered into all 8 destinations' 8192x4096 bf16 windows.
GEMM_AR_MLP = GemmRS("gemm_ar_mlpdown_p8_8192x4096x1792_bf16", P=8, M=8192, N=4096, K=1792,
                     in_dt=BF16, slot_dt=F32, out_dt=BF16, tile_m=256, tile_n=256)



@dataclass(frozen=True)
class GemmA2A:
    name: str
    P: int          # ranks
    E: int          # experts per rank (P * E in all)
    B: int          # tokens per rank
    topk: int       # experts per token
    N: int          # model width (output of the expert's down projection)
    K: int          # expert hidden width
    cap: int        # rows of each destination window
    tile_m: int = 256   # expert groups are padded to whole tiles of this many rows
    tile_n: int = 256


# GEMM+All-to-All, the MoE combine: 8 ranks x 4096 tokens, top-2 of 32 experts;
# this rank's 4 experts project 1792 -> 4096 and send each row to its token's rank
# (about 1024 rows per destination; windows hold twice that).
GEMM_A2A_MOE = GemmA2A("gemm_a2a_moe_p8_e4_b4096_top2_1792x4096_bf16", P=8, E=4, B=4096, topk=2,
                       N=4096, K=1792, cap=2048)

ALL = [GEMM_RS_TINY, GEMV_AR_DECODE, GEMM_RS_MLP, AG_GEMM_COL, EMBBAG_DLRM]


@dataclass(frozen=True)
class A2aGemm:
    name: str
    P: int          # source ranks
    E: int          # experts per rank (P * E in all); this rank owns experts 0 .. E-1
    B: int          # tokens per source rank
    topk: int       # experts per token
    N: int          # expert hidden width (output of the up projection)
    K: int          # model width
    cap: int        # rows of the receive buffer
    tile_m: int = 256
    tile_n: int = 256


# All-to-All + GEMM, the MoE dispatch: 8 ranks x 4096 tokens, top-2 of 32 experts; the rows
# routed to this rank's 4 experts arrive grouped by expert and are projected 4096 -> 1792
# (the up projection; the GEMM + All-to-All combine above is the matching down projection).
A2A_GEMM_MOE = A2aGemm("a2a_gemm_moe_p8_e4_b4096_top2_4096x1792_bf16", P=8, E=4, B=4096, topk=2,
                       N=1792, K=4096, cap=12288)
