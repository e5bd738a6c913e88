"""W12 on MI355X: lossless 12-bit BF16 weights and the decode-in-register skinny GEMM.

The compute lives in libw12.so (hand-written HIP for gfx950, C ABI in include/w12.h);
this package only marshals arguments to it.
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    W12Error,
    W12Tensor,
    alloc_planes,
    bits_per_weight,
    decode,
    encode,
    encode_count,
    encode_emit,
    encode_many,
    file_index,
    GROUP_INLINE,
    GROUP_MAX,
    gemm,
    gemm_noalloc,
    gemm_group,
    gemm_group_workspace,
    gemm_group_workspace_size,
    gemm_plan,
    gemm_workspace,
    gemm_workspace_init,
    gemm_workspace_size,
    layout_bytes,
    tensor_bytes,
    lib,
    load,
    read_probe,
    save,
    unpack_records,
    verify,
    verify_async,
)
