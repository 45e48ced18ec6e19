/* A plain C caller of the C-ABI: compiles against include/int8attn.h alone, links
 * libint8attn.so, and checks the host-side contract without a GPU: the version, and
 * that invalid arguments come back as the documented error codes with a message (every
 * call below is rejected before any device work). Prints "c-abi ok" on success. */
#include <stdio.h>
#include <string.h>

#include "int8attn.h"

#define FAKE ((void*)0x1000)

static int fails = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: got %d, want %d (%s)\n", what, got, want, int8attn_last_error());
    ++fails;
  }
}

int main(void) {
  if (int8attn_version() <= 0) {
    printf("FAIL version %d\n", int8attn_version());
    ++fails;
  }
  /* head_dim other than 256 */
  expect("kv_quant_write head_dim", kv_quant_write(FAKE, FAKE, I8A_DTYPE_F32, 4, 4, 128, FAKE, FAKE,
                                                   FAKE, FAKE, FAKE, 16, NULL),
         I8A_EUNSUPPORTED);
  if (strlen(int8attn_last_error()) == 0) {
    printf("FAIL no error message\n");
    ++fails;
  }
  /* unknown dtype flag */
  expect("kv_quant_write dtype", kv_quant_write(FAKE, FAKE, 7, 4, 4, 256, FAKE, FAKE, FAKE, FAKE,
                                                FAKE, 16, NULL),
         I8A_EINVAL);
  /* decode workspace too small */
  {
    size_t need = attn_decode_workspace_bytes(2, 1000, 24, 256);
    expect("decode workspace size", need > 0, 1);
    expect("decode workspace", attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 63, FAKE, 2, 1000,
                                           16, 24, 4, 256, 0.0625f, FAKE, FAKE, need - 1, NULL),
           I8A_EWORKSPACE);
  }
  /* prefill: n_new past the context */
  expect("prefill n_new", attn_prefill_chunk(FAKE, 101, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1, 16, 24,
                                             4, 256, 0.0625f, FAKE, NULL),
         I8A_EINVAL);
  /* split prefill: workspace not 16-byte aligned */
  {
    size_t need = attn_prefill_chunk_split_workspace_bytes(16, 100, 1, 24, 4, 256);
    expect("split workspace size", need > 0, 1);
    expect("split alignment", attn_prefill_chunk_split(FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1,
                                                       16, 24, 4, 256, 0.0625f, FAKE,
                                                       (char*)FAKE + 4, need, NULL),
           I8A_EINVAL);
  }
  /* no work: a no-op that succeeds */
  expect("prefill n_new 0", attn_prefill_chunk(FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1, 16, 24,
                                               4, 256, 0.0625f, FAKE, NULL),
         I8A_OK);
  if (fails) return 1;
  printf("c-abi ok\n");
  return 0;
}
