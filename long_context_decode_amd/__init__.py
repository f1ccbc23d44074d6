"""Compressed-KV decode attention on AMD MI355X (gfx950).

Thin Python binding of the C ABI in ``include/lcd.h`` (``liblcd.so``): argument
marshalling only.  torch supplies device memory and streams; every step of the
decode and compression path runs in the library's HIP kernels.  Importing this
package fails loudly if the library has not been built
(``python long_context_decode_amd/build.py``).
"""
from ._lib import (  # noqa: F401
    LCD_APPEND,
    LCD_BF16,
    LCD_F32,
    LCD_H2O,
    LCD_DUO,
    LCD_SINK_RING,
    LIB_PATH,
    KVCache,
    LcdError,
    abi_version,
    cache_config,
    cache_sizes,
    decode_attn,
    decode_step,
    decode_step_noalloc,
    kv_append,
    kv_cache_destroy,
    kv_cache_init,
    kv_filled,
    kv_layer_bytes,
    kv_layer_view,
    kv_load,
    kv_save,
    LayerState,
    kv_rank_of,
    kv_set_filled,
    kv_slot_of,
    kv_tokens,
    pyramid_budgets,
    h2o_prompt_params,
    h2o_prompt_sizes,
    h2o_prompt_compress,
    last_error,
    lib,
    snapkv_compress,
    snapkv_params,
    snapkv_sizes,
)
