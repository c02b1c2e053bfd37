// Exercises the host side of libmoe's entry points -- argument validation, workspace layout,
// capacity and size queries -- with arguments that are rejected before anything is enqueued,
// so that a build of that code with AddressSanitizer and UndefinedBehaviorSanitizer checks it
// without a GPU.  Prints "abi-sanitize ok" and exits 0 when every status is as expected.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/moe.h"

#define CHECK(cond) do { if (!(cond)) { fprintf(stderr, "check failed: %s (line %d): %s\n", #cond, __LINE__, moe_last_error()); exit(1); } } while (0)

static void* fake(uintptr_t v) { return (void*)v; }  // never dereferenced: validation fails first

int main() {
  // route / sort / quant: bad arguments
  CHECK(moe_route_topk((const float*)fake(0x1000), 4, 0, 1, MOE_SCORE_SOFTMAX, 1, 0, 1.0f, nullptr, nullptr, nullptr) == MOE_EINVAL);
  CHECK(strlen(moe_last_error()) > 0);
  CHECK(moe_route_topk(nullptr, 4, 8, 2, MOE_SCORE_SOFTMAX, 1, 0, 1.0f, nullptr, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_route_grouped_topk((const float*)fake(0x1000), nullptr, 4, 12, 2, 5, 2, MOE_SCORE_SIGMOID, 1, 1.0f, 0, 1.0f,
                               (int32_t*)fake(0x2000), (float*)fake(0x3000), nullptr) == MOE_EINVAL);
  CHECK(moe_map_experts(nullptr, nullptr, nullptr, 4, 0, 8, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_align_sort(nullptr, 4, 2, 8, 48, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_route_align(nullptr, 4, 8, 2, MOE_SCORE_SOFTMAX, 1, 0, 1.0f, 16, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_quant_act(nullptr, 4, 33, MOE_A_FP8_G128, nullptr, nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_quant_act(nullptr, 4, 64, MOE_A_BF16, nullptr, nullptr, nullptr) == MOE_EINVAL);
  // sizes and queries
  CHECK(moe_sort_capacity(64, 4, 32, 16) == 64 * 4 + 32 * 15);
  CHECK(moe_sort_capacity(-1, 4, 32, 16) == 0);
  CHECK(moe_tiled_weight_bytes(MOE_W_MXFP4, 2, 64, 256) == 2 * 4 * 2 * 1088);
  CHECK(moe_tiled_weight_bytes(MOE_W_FP8_BLOCK128, 2, 60, 256) == 0);
  CHECK(moe_supports(MOE_W_MXFP4, MOE_A_BF16, MOE_ACT_SILU, 2880, 2880) == MOE_OK);
  CHECK(moe_supports(MOE_W_MXFP4, MOE_A_FP8_G128, MOE_ACT_SILU, 2880, 2880) == MOE_EUNSUPPORTED);
  CHECK(moe_supports(MOE_W_FP8_BLOCK128, MOE_A_FP8_G128, MOE_ACT_SILU, 100, 2880) == MOE_EINVAL);
  for (int T = 0; T < 9000; T += 997) {
    const int bm = moe_pick_block_m(T, 4, 128, MOE_W_FP8_BLOCK128, MOE_LAYOUT_TILED);
    CHECK(bm == 16 || bm == 32 || bm == 64 || bm == 128);
  }
  CHECK(moe_tile_weights(MOE_W_MXFP4, 2, 60, 256, nullptr, nullptr, nullptr, nullptr) == MOE_EINVAL);
  // the forward: layout of every format pair, then rejected calls
  const moe_wfmt wf[6] = {MOE_W_MXFP4, MOE_W_MXFP4, MOE_W_FP8_BLOCK128, MOE_W_FP8_CHANNEL, MOE_W_FP8_TENSOR, MOE_W_BF16};
  const moe_afmt af[6] = {MOE_A_BF16, MOE_A_MXFP4_G32, MOE_A_FP8_G128, MOE_A_FP8_TOKEN, MOE_A_FP8_TENSOR, MOE_A_BF16};
  for (int f = 0; f < 6; ++f) {
    for (int bm = 16; bm <= 128; bm *= 2) {
      moe_forward_args a;
      memset(&a, 0, sizeof a);
      a.T = 4096; a.H = 7168; a.I = 2048; a.E_total = 257; a.K = 9; a.block_m = bm;
      a.wfmt = wf[f]; a.afmt = af[f]; a.act = MOE_ACT_SILU;
      moe_workspace_layout_t L;
      const moe_status st = moe_workspace_layout(&a, &L);
      if (wf[f] == MOE_W_BF16 && (bm == 32 || bm == 16)) {
        CHECK(st == MOE_EUNSUPPORTED);
        continue;
      }
      CHECK(st == MOE_OK);
      CHECK(L.total == moe_experts_workspace_bytes(&a) && L.total >= L.ybuf_off + L.ybuf_bytes);
      CHECK(L.h_bytes == moe_sort_capacity(a.T, a.K, a.E_total, bm) * (size_t)a.I * 2);
      CHECK(moe_experts_forward(&a, nullptr) == MOE_EINVAL);                 // NULL tensors
      CHECK(moe_experts_forward_noalloc(&a, nullptr) == MOE_EWORKSPACE);     // beyond the scratch
      CHECK(moe_layer_forward(&a, nullptr, MOE_SCORE_SOFTMAX, 1, 0, 1.0f, nullptr, nullptr, nullptr) == MOE_EINVAL);
      a.H = 7000;
      CHECK(moe_experts_forward(&a, nullptr) == MOE_EINVAL);
      CHECK(moe_workspace_layout(&a, &L) == MOE_EINVAL);
    }
  }
  moe_forward_args z;
  memset(&z, 0, sizeof z);
  CHECK(moe_experts_forward(nullptr, nullptr) == MOE_EINVAL);
  CHECK(moe_experts_forward(&z, nullptr) == MOE_EINVAL);
  CHECK(moe_profile_events(nullptr, 3) == MOE_EINVAL);
  CHECK(moe_profile_events(nullptr, 0) == MOE_OK);
  CHECK(moe_set_checked_mode(1) == MOE_OK);  // host state only; the check itself runs on a forward call
  CHECK(moe_set_checked_mode(0) == MOE_OK);
  CHECK(moe_last_error()[0] == '\0');
  printf("abi-sanitize ok\n");
  return 0;
}
