// Drives the host side of the KDA C ABI (argument checks, launch-shape choice,
// the duplicate-slot debug check, workspace sizes, status text) in a build with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code. Device
// pointers are fake, 256-byte aligned addresses that the host never
// dereferences; every call below either fails a host check or reaches the
// launch, which fails without a GPU (KDA_ERR_HIP) or, on a machine with one,
// is never reached because each case fails a check first. Run only where no
// GPU is visible. Exits 0 when every status is the one expected.
#include <stdint.h>
#include <stdio.h>

#include "kda.h"

#define CHECK(expr, want)                                                                 \
  do {                                                                                    \
    const int got_ = (expr);                                                              \
    if (got_ != (want)) {                                                                 \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, want); \
      return 1;                                                                           \
    }                                                                                     \
  } while (0)

int main() {
  float *const F = reinterpret_cast<float *>(0x10000);
  const uint16_t *const U = reinterpret_cast<const uint16_t *>(0x10000);
  const int32_t *const I = reinterpret_cast<const int32_t *>(0x10000);
  const int64_t stride = 2 * 128 * 128;
  kda_options none = {0, 0, 0}, bad_flag = {0, 0, 8}, chk = {0, 0, KDA_CHECK_SLOTS}, tile3 = {3, 0, 0};
  const int32_t dup[4] = {3, 1, -1, 3}, ok[4] = {3, -1, 1, -1};

  // decode
  CHECK(kda_decode_step(F, 8, stride, I, 0, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, &none, nullptr), KDA_OK);
  CHECK(kda_decode_step(F, 8, stride, I, -1, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, nullptr, nullptr),
        KDA_ERR_INVALID);
  CHECK(kda_decode_step(F, 8, stride, I, 4, 2, 96, 128, U, U, U, F, F, F, nullptr, nullptr, nullptr, nullptr),
        KDA_ERR_UNSUPPORTED);
  CHECK(kda_decode_step(F, 8, stride, I, 4, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, &bad_flag, nullptr),
        KDA_ERR_INVALID);
  CHECK(kda_decode_step(F, 8, stride, I, 4, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, &tile3, nullptr),
        KDA_ERR_UNSUPPORTED);
  CHECK(kda_decode_step(F, 8, stride, dup, 4, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, &chk, nullptr),
        KDA_ERR_INVALID);
  CHECK(kda_decode_step(F, 8, stride, ok, 4, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, &chk, nullptr),
        KDA_ERR_HIP);
  CHECK(kda_decode_step(F, 8, stride - 4, I, 4, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, nullptr, nullptr),
        KDA_ERR_INVALID);
  kda_epilogue bad_eps = {U, nullptr, -1.0f};
  CHECK(kda_decode_step(F, 8, stride, I, 4, 2, 128, 128, U, U, U, F, F, F, &bad_eps, nullptr, nullptr, nullptr),
        KDA_ERR_INVALID);

  // verify, commit
  kda_replay_buf rb = {const_cast<uint16_t *>(U), const_cast<uint16_t *>(U), F, F};
  for (int mode = 0; mode < 2; ++mode) {
    CHECK(kda_verify_chunk(F, 8, stride, dup, I, 4, 4, 9, 2, 128, 128, U, U, U, F, F, F, nullptr, mode, 0, &rb, F,
                           nullptr, &chk, nullptr),
          KDA_ERR_INVALID);
    CHECK(kda_verify_chunk(F, 8, stride, ok, I, 4, 4, 9, 2, 128, 128, U, U, U, F, F, F, nullptr, mode, 0, &rb, F,
                           nullptr, &chk, nullptr),
          KDA_ERR_HIP);
    CHECK(kda_replay_commit(F, 8, stride, dup, nullptr, I, 4, 4, 0, 2, 128, 128, mode, &rb, F, nullptr, &chk,
                            nullptr),
          KDA_ERR_INVALID);
    CHECK(kda_replay_commit(F, 8, stride, ok, nullptr, I, 4, 4, 0, 2, 128, 128, mode, &rb, F, nullptr, &chk,
                            nullptr),
          KDA_ERR_HIP);
  }
  CHECK(kda_verify_chunk(F, 8, stride, I, I, 4, 17, 9, 2, 128, 128, U, U, U, F, F, F, nullptr, 0, 0, &rb, nullptr,
                         nullptr, nullptr, nullptr),
        KDA_ERR_UNSUPPORTED);
  CHECK(kda_verify_chunk(F, 8, stride, I, I, 4, 4, 9, 2, 128, 128, U, U, U, F, F, F, nullptr, 0, 0, nullptr,
                         nullptr, nullptr, nullptr, nullptr),
        KDA_ERR_INVALID);

  // prefill, both forms, and the static-scratch form
  const int32_t pos[4] = {0, 1, -1, 2};
  CHECK(kda_prefill(F, 8, stride, dup, I, 4, 90, 2, 128, 128, U, U, U, F, F, F, pos, F, nullptr, &chk, nullptr),
        KDA_ERR_INVALID);
  CHECK(kda_prefill(F, 8, stride, ok, I, 4, 90, 2, 128, 128, U, U, U, F, F, F, pos, F, nullptr, &chk, nullptr),
        KDA_ERR_HIP);
  size_t ws = 0;
  CHECK(kda_prefill_chunked_workspace(4, 90, 2, 128, 128, &ws), KDA_OK);
  CHECK(kda_prefill_chunked(F, 8, stride, I, I, 4, 90, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, F, ws - 1,
                            nullptr, nullptr, nullptr),
        KDA_ERR_INVALID);
  CHECK(kda_prefill_chunked(F, 8, stride, ok, I, 4, 90, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr, F, ws,
                            nullptr, &chk, nullptr),
        KDA_ERR_HIP);
  CHECK(kda_prefill_chunked_noalloc(F, 8, 32 * 128 * 128, ok, I, 1, 1 << 20, 32, 128, 128, U, U, U, F, F, F,
                                    nullptr, nullptr, nullptr, nullptr, nullptr),
        KDA_ERR_TOO_LARGE);
  CHECK(kda_prefill_chunked_noalloc(F, 8, stride, dup, I, 4, 90, 2, 128, 128, U, U, U, F, F, F, nullptr, nullptr,
                                    nullptr, &chk, nullptr),
        KDA_ERR_INVALID);

  // state transfer, launch shapes, status text
  CHECK(kda_state_pack(F, 8, stride, I, 4, 2, 128, 128, 1, 2, 0, 128, F, nullptr, nullptr), KDA_ERR_INVALID);
  CHECK(kda_state_unpack(F, 8, stride, I, 4, 2, 128, 128, 0, 2, 100, 64, F, nullptr, nullptr), KDA_ERR_INVALID);
  int32_t w = 0, t = 0;
  for (int op = 0; op < 5; ++op)
    for (int B = 1; B <= 4096; B *= 2)
      for (int H = 1; H <= 64; H *= 4) CHECK(kda_query_variant(op, B, H, 128, 128, 8, 0, 0, &w, &t), KDA_OK);
  CHECK(kda_query_variant(9, 1, 1, 128, 128, 1, 0, 0, &w, &t), KDA_ERR_INVALID);
  for (int s = -6; s <= 1; ++s)
    if (!kda_status_str(s)) return 1;
  printf("abi driver: ok\n");
  return 0;
}
