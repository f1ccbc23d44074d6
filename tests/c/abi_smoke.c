/* Plain C99 client of the C ABI: include/lcd.h must compile as C, every entry point it
 * declares must link against liblcd.so, and calls that fail validation must return an
 * error status without touching a device (no GPU is needed to run this). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lcd.h"

int main(void) {
  if (lcd_abi_version() != LCD_ABI_VERSION) {
    printf("abi version %d != header %d\n", lcd_abi_version(), LCD_ABI_VERSION);
    return 1;
  }
  /* a null handle is rejected before any HIP call */
  if (lcd_decode_attn(NULL, 0, NULL, NULL, NULL, 0, NULL) == LCD_OK) return 2;
  if (lcd_decode_step(NULL, 0, NULL, NULL, NULL, NULL, NULL, 0, NULL) == LCD_OK) return 3;
  if (lcd_kv_append(NULL, 0, NULL, NULL, 1, NULL) == LCD_OK) return 4;
  /* a bad configuration is rejected by the size query */
  lcd_cache_config cfg;
  memset(&cfg, 0, sizeof cfg);
  uint64_t kv = 0, aux = 0, ws = 0;
  if (lcd_cache_sizes(&cfg, &kv, &aux, &ws) == LCD_OK) return 5;
  const char* msg = lcd_last_error();
  if (!msg || !msg[0]) return 6;
  printf("ok: abi %d, last error \"%s\"\n", lcd_abi_version(), msg);
  return 0;
}
