"""Workload shapes (innermost-first dims, byte strides, boxes) and seeds.

Sizes follow the reference pages' worked examples and the benchmark
configurations; they are data only.
"""

# Worked example (a): 16 x 128 fp16 tensor, 8 x 64 box, swizzle NONE / 128B.
EXAMPLE_2D = dict(dtype="f16", dims=(128, 16), strides=(256,), box=(64, 8),
                  coords=((0, 0), (64, 8)), seed=1)

# Worked example (b): 16 x 256 fp16 matrix viewed as (group, row, col); one
# 3D box of 2 x 16 x 64 per 128-column slice -> four 8 x 128-byte atoms.
EXAMPLE_3D = dict(dtype="f16", dims=(64, 16, 4), strides=(512, 128), box=(64, 16, 2),
                  coords=((0, 0, 0), (0, 0, 2)), seed=1)

# Round-trip copy: bf16 8192 x 8192, box 128 rows x 64 columns, 128B swizzle.
COPY_8192 = dict(dtype="bf16", dims=(8192, 8192), strides=(16384,), box=(64, 128),
                 swizzle="128b", seed=2)

# Rank-5 fp32 with element strides and edge-crossing boxes.
RANK5 = dict(dtype="f32", dims=(260, 129, 33, 7, 3), box=(32, 32, 8, 2, 1),
             estride=(1, 2, 1, 1, 1), swizzle="128b", nbox=2048, seed=3)

# Reduce-store: 4096 x 4096 destination, 4 passes of 1024 boxes of 64 x 64.
REDUCE_4096 = dict(dims=(4096, 4096), strides=(16384,), box=(64, 64), passes=4,
                   nbox=1024, seed=4)

# GEMM consumer: M = N = K = 8192, A row-major, B column-major.
GEMM_8192 = dict(M=8192, N=8192, K=8192, tile_m=256, tile_n=256, tile_k=64,
                 nsample=4096, seed=5)

WORKLOADS = dict(example_2d=EXAMPLE_2D, example_3d=EXAMPLE_3D, copy_8192=COPY_8192,
                 rank5=RANK5, reduce_4096=REDUCE_4096, gemm_8192=GEMM_8192)
