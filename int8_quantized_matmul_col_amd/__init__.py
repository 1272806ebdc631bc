"""LLM.int8() mixed-precision decomposed matmul for AMD Instinct MI355X (gfx950).

    Y = X_O . W_O (fp16) + dequant(int8(X_R) . int8(W_R))

The computation lives in hand-written HIP kernels behind a C ABI
(``include/int8mm.h``, built into ``libint8mm.so``); this package is the thin
Python binding over it, with torch used only for device memory and streams.

    import int8_quantized_matmul_col_amd as mm
    Wq, w_scale = mm.int8_prepare_weight(W)          # once per weight
    Y = mm.int8_matmul(X, Wq, w_scale, threshold=6.0)
    Y = mm.int8_linear(X, Wq, w_scale, bias)          # with a layer's bias

``Int8Linear`` wraps the same calls as a torch module (forward only), and
``replace_linear_with_int8`` swaps the fp16 ``nn.Linear`` layers of a model
for it.  ``outlier_stats`` summarizes the column maxima of an activation
(``int8_column_absmax``) and |O| at candidate thresholds
(``int8_outlier_counts``) to help choose the threshold.
"""

from .binding import (  # noqa: F401
    DEFAULT_THRESHOLD,
    INT8MM_DECODE_MAX_M,
    INT8MM_MAX_K,
    Int8mmError,
    int8_column_absmax,
    int8_linear,
    int8_matmul,
    int8_matmul_noalloc,
    int8_matmul_noalloc_max_workspace,
    int8_matmul_profiled,
    int8_matmul_stages,
    int8_matmul_workspace_size,
    int8_outlier_counts,
    int8_pack_weight,
    int8_prepare_weight,
    int8_weight_bytes,
    int8_weight_ld,
    padded_rows,
    unpack_weight,
    untile,
    load,
    workspace_for,
)
from .linear import Int8Linear, replace_linear_with_int8  # noqa: F401
from .stats import outlier_stats, suggest_threshold  # noqa: F401
