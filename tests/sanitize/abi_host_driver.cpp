// Host-only driver of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side of every library source
// (tests/test_host_sanitizers.py). It runs every path that returns before
// any HIP call: the argument checks of each entry point, the workspace plan
// over the whole size envelope, the status strings and the workspace check.
// Exit status 0 when every expectation holds; a sanitizer report aborts.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "moe_decode.h"

static int failures = 0;

#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

int main() {
  // Workspace sizes over the envelope (and just outside it).
  const int Bs[] = {1, 2, 16, 64, 255, 256, 257};
  const int ds[] = {8, 256, 2048, 4096, 16384, 16392};
  const int Es[] = {1, 16, 128, 256, 257};
  const int Is[] = {8, 768, 1536, 16384};
  const int ks[] = {1, 8, 16, 17};
  size_t prev = 0;
  int n_ok = 0;
  for (int B : Bs)
    for (int d : ds)
      for (int E : Es)
        for (int I : Is)
          for (int k : ks)
            for (int dt = 0; dt < 2; ++dt) {
              const size_t w = moe_workspace_bytes(B, d, E, I, k, dt ? MOE_BF16 : MOE_F32);
              const bool inside = B <= 256 && d <= 16384 && E <= 256 && k <= 16 && k <= E;
              EXPECT(inside == (w != 0));
              if (w) {
                EXPECT(w % 256 == 0);
                EXPECT(w >= MOE_WS_STATUS_BYTES);
                ++n_ok;
              }
              prev ^= w;
            }
  EXPECT(n_ok > 0);
  // Bigger batches never need less workspace.
  for (int B = 1; B < 256; ++B)
    EXPECT(moe_workspace_bytes(B, 2048, 128, 768, 8, MOE_BF16) <= moe_workspace_bytes(B + 1, 2048, 128, 768, 8, MOE_BF16));

  // Status strings, including an unknown code.
  for (int s = 0; s <= 8; ++s) {
    const char *t = moe_status_string(static_cast<moe_status_t>(s));
    EXPECT(t != nullptr && strlen(t) > 0);
  }

  // Workspace check on host copies of the status bytes.
  std::vector<unsigned char> st(MOE_WS_STATUS_BYTES, 0);
  EXPECT(moe_workspace_check(st.data(), st.size()) == MOE_OK);
  st[256] = 1;
  EXPECT(moe_workspace_check(st.data(), st.size()) == MOE_ERR_SYNC_TIMEOUT);
  EXPECT(moe_workspace_check(st.data(), st.size() - 1) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_workspace_check(nullptr, st.size()) == MOE_ERR_INVALID_ARG);

  // Argument checks: host addresses stand in for device pointers (no call
  // below gets past its checks, so none is dereferenced).
  alignas(256) static unsigned char buf[4096];
  void *p = buf;
  int32_t *ip = reinterpret_cast<int32_t *>(buf);
  float *fp = reinterpret_cast<float *>(buf);
  moe_routing_t r{ip, fp, ip, ip, ip, ip, ip, fp};
  moe_routing_t r_null = r;
  r_null.pair_slot = nullptr;
  const moe_policy_t topk{MOE_POLICY_TOPK, 8, 0, 0, 0};
  const moe_policy_t bad_oea{MOE_POLICY_OEA, 8, 9, 0, 0};
  const moe_policy_t bad_kind{42, 8, 0, 0, 0};
  const moe_policy_t bad_lynx{MOE_POLICY_LYNX, 8, 0, 4, 0};
  const moe_policy_t bad_hier{MOE_POLICY_HIER, 8, 5, 4, 1};

  EXPECT(moe_route(nullptr, p, nullptr, MOE_BF16, 16, 2048, 128, fp, p, 1 << 20, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route(p, p, nullptr, MOE_BF16, 0, 2048, 128, fp, p, 1 << 20, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_route(p, p, nullptr, MOE_BF16, 300, 2048, 128, fp, p, 1 << 20, nullptr) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route(p, p, nullptr, MOE_BF16, 16, 2048, 128, fp, p, 16, nullptr) == MOE_ERR_WORKSPACE);
  EXPECT(moe_route(p, p, nullptr, static_cast<moe_dtype_t>(7), 16, 2048, 128, fp, p, 1 << 20, nullptr) ==
         MOE_ERR_INVALID_ARG);

  EXPECT(moe_select(nullptr, 16, 128, topk, &r, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_select(fp, 16, 128, bad_oea, &r, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_select(fp, 16, 128, bad_kind, &r, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_select(fp, 16, 128, bad_lynx, &r, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_select(fp, 16, 128, bad_hier, &r, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_select(fp, 16, 128, topk, &r_null, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_select(fp, 16, 128, topk, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_select(fp, 300, 128, topk, &r, nullptr) == MOE_ERR_UNSUPPORTED);

  const size_t ws = moe_workspace_bytes(16, 2048, 128, 768, 8, MOE_BF16);
  EXPECT(moe_expert_ffn(p, p, p, p, MOE_BF16, 16, 2048, 128, 768, 8, &r, p, p, ws - 256, nullptr) ==
         MOE_ERR_WORKSPACE);
  EXPECT(moe_expert_ffn(p, p, p, p, MOE_BF16, 16, 2048, 128, 768, 8, &r, p, nullptr, ws, nullptr) ==
         MOE_ERR_WORKSPACE);
  EXPECT(moe_expert_ffn(buf + 4, p, p, p, MOE_BF16, 16, 2048, 128, 768, 8, &r, p, p, ws, nullptr) ==
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_expert_ffn(p, p, p, p, MOE_BF16, 16, 2044, 128, 768, 8, &r, p, p, ws, nullptr) ==
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_expert_ffn(p, p, p, p, MOE_BF16, 16, 2048, 4, 768, 8, &r, p, p, ws, nullptr) ==
         MOE_ERR_INVALID_ARG);

  EXPECT(moe_layer_decode(p, p, nullptr, p, p, p, MOE_BF16, 16, 2048, 128, 768, bad_oea, fp, &r, p, p, ws,
                          nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_decode(p, p, nullptr, p, p, p, MOE_BF16, 16, 2048, 128, 768, topk, fp, &r, p, p, 256,
                          nullptr) == MOE_ERR_WORKSPACE);
  EXPECT(moe_layer_decode(p, p, nullptr, p, p, p, MOE_BF16, 16, 2048, 128, 768, topk, nullptr, &r, p, p, ws,
                          nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_layer_decode_static(p, p, nullptr, p, p, p, MOE_BF16, 256, 16384, 256, 16384, topk, fp, &r, p,
                                 nullptr) == MOE_ERR_SCRATCH);
  EXPECT(moe_layer_decode_static(p, p, nullptr, p, p, p, MOE_BF16, 16, 2048, 128, 768, bad_kind, fp, &r, p,
                                 nullptr) == MOE_ERR_INVALID_ARG);

  EXPECT(moe_read_stream(p, 0, reinterpret_cast<uint32_t *>(buf), nullptr) == MOE_ERR_INVALID_ARG);
  EXPECT(moe_read_stream(p, 24, reinterpret_cast<uint32_t *>(buf), nullptr) == MOE_ERR_INVALID_ARG);

  printf("abi host driver: %d failures, %d workspace sizes inside the envelope (%zx)\n", failures, n_ok, prev);
  return failures ? 1 : 0;
}
